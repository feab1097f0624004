// Block-causal attention over the cached history plus the unit's own tokens,
// split over the key axis ("通义实验室发布 Wan-Streamer v0.2…", section
// 为什么端到端模型对级联式 AI 智能体构成挑战: each streaming block may only see
// what is already available, so no output depends on later frames; query
// unit u sees every key of units <= u, bidirectionally inside unit u).
//
// Design for gfx950 (CDNA4), one workgroup = 4 waves = 128 query rows of one
// head and one contiguous chunk ("split") of that head's visible keys:
//
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    K (32 keys x 16 dims) is the A operand read from LDS, Q^T the B operand
//    held in registers for the whole kernel. In the accumulator layout every
//    lane then owns one query row (lane % 32) and 16 of a 32-key block's keys,
//    so the row max is a per-lane max plus one exchange with lane ^ 32, and
//    the probabilities are already in the B-operand layout of O^T = V^T P^T:
//    P never leaves registers.
//  * V is staged in LDS transposed (V^T, dims x keys) with the keys of each
//    16-key group permuted (bits 2 and 3 of the key index swapped) so that a
//    lane's eight B-operand keys of P are contiguous in V^T: the A operand of
//    the PV product is one 16-byte LDS read. The transpose happens once per
//    tile while writing LDS (4-key x 8-dim register blocks, v_perm).
//  * Online softmax in the exp2 domain, fp32, with the running max allowed to
//    lag the true max by up to 2^8 before O and l are rescaled (rescales are
//    rare once the max settles; the result is the same up to rounding).
//  * Software pipeline over 64-key tiles: while the vector unit runs the
//    softmax of tile t, the matrix cores already compute S^T of tile t+1, then
//    O^T += V^T P^T of tile t. K and V^T each have two LDS stages (72 KB at
//    D = 128, so two workgroups fit in a CU's 160 KB); K is written two tiles
//    ahead and V one tile ahead, which needs one barrier per tile. Global
//    loads are issued a tile before use. A tile never straddles the cache and
//    the own tokens; its rows are read with raw buffer loads at per-thread
//    constant offsets from a resource built per tile with scalar instructions,
//    whose range ends at the tile's last valid row (zeros past it).
//  * Work items (head, split, query tile) are ordered with the query tile
//    fastest and mapped onto blockIdx so that the items of one (head, split)
//    land on the same XCD (workgroups are dispatched round-robin over the 8
//    XCDs): the K/V chunk they share is then served from that XCD's L2.
//  * Rows past the visible range read as zeros and are masked to -inf, so
//    unused cache capacity never reaches the arithmetic.
#include <math.h>

#include "ws_device.hpp"
#include "ws_launch.hpp"

namespace ws {
namespace {

constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag
constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
struct Tile {
  static constexpr int kKPitch = D + 8;              // bf16 per K row in LDS
  static constexpr int kVPitch = kAttnBlockN + 8;    // bf16 per V^T row
  static constexpr int kKElems = kAttnBlockN * kKPitch;
  static constexpr int kVElems = D * kVPitch;
  static constexpr int kStage = kKElems + kVElems;
  static constexpr int kKChunks = kAttnBlockN * (D / 8) / kThreads;  // per thread
  static constexpr int kVTasks = (kAttnBlockN / 4) * (D / 8);         // 4 keys x 8 dims each
  static constexpr int kDSteps = D / 16;   // k-steps of the QK^T product
  static constexpr int kDBlocks = D / 32;  // 32-dim blocks of O^T
  static_assert(kKChunks * kThreads == kAttnBlockN * (D / 8), "K tile split");
  static_assert(kVTasks <= kThreads, "V tile split");
};

// Position of a key (within a 64-key tile) in a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int key) {
  const int b = ((key >> 2) ^ (key >> 3)) & 1;
  return key ^ (b * 12);
}

// Visible-key count of a query row from the unit table.
__device__ __forceinline__ int row_kend(const AttnArgs& a, int row) {
  int u = 0;
  while (u + 1 < a.n_units && a.q_unit_begin[u + 1] <= row) ++u;
  return a.unit_kend[u];
}


template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_partial_kernel(const AttnArgs a) {
  using T = Tile<D>;
  // two K stages then two V^T stages
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::kKElems + 2 * T::kVElems];

  // ---- work item: XCD-aware decode of (head, split, query tile)
  const int per_xcd = gridDim.x >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= a.n_items) return;
  const int qt = w % a.n_qtiles;
  const int hs = w / a.n_qtiles;
  const int split = hs % a.n_splits;
  const int h = hs / a.n_splits;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  const int r0 = qt * kAttnBlockM;
  const int r_last = min(r0 + kAttnBlockM, a.n_q) - 1;
  const int kmin = row_kend(a, r0);     // smallest visible range in this tile
  const int kmax = row_kend(a, r_last);  // largest (kend is non-decreasing)
  // tiles: cache rows [0, min(len, kmax)) then own tokens [len, kmax)
  const int cache_rows = min(a.len, kmax);
  const int self_rows = max(0, kmax - a.len);
  const int n_ct = (cache_rows + kAttnBlockN - 1) / kAttnBlockN;
  const int n_kt = n_ct + (self_rows + kAttnBlockN - 1) / kAttnBlockN;
  const int t_begin = (int)((int64_t)split * n_kt / a.n_splits);
  const int n_t = (int)((int64_t)(split + 1) * n_kt / a.n_splits) - t_begin;

  const uint16_t* kc_h = a.kc + h * a.cache_head_stride;
  const uint16_t* vc_h = a.vc + h * a.cache_head_stride;
  const uint16_t* ks_h = a.ks + (int64_t)h * a.n_self * D;
  const uint16_t* vs_h = a.vs + (int64_t)h * a.n_self * D;

  // ---- this lane's query row and its Q^T operands
  const int qrow = r0 + wave * 32 + lrow;
  const bool wave_active = r0 + wave * 32 < a.n_q;
  // the unit of a row is the last non-empty unit starting at or before it;
  // the loop index is uniform, so the table is read with scalar loads
  int kend = 0;
  for (int u = 0; u < a.n_units; ++u) kend = qrow >= a.q_unit_begin[u] ? a.unit_kend[u] : kend;
  if (qrow >= a.n_q) kend = 0;
  u32x4 qf[T::kDSteps];
  {
    const uint16_t* qp = a.q + ((int64_t)h * a.n_q + qrow) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
      qf[ks] = qrow < a.n_q ? *reinterpret_cast<const u32x4*>(qp + ks * 16) : u32x4{0, 0, 0, 0};
    // wait for Q here, once: otherwise paths that skip the prologue leave the
    // loads pending and every tile's first MFMA would wait on all loads
    __builtin_amdgcn_s_waitcnt(0);
  }

  f32x16 o[T::kDBlocks];
#pragma unroll
  for (int db = 0; db < T::kDBlocks; ++db) o[db] = f32x16{};
  float m_run = kNegInf;  // running max of scaled scores (log2 units)
  float l_run = 0.f;      // this lane's share of the softmax denominator

  // ---- per-thread constant offsets of the tile staging
  // K: rows kKChunks*(tid / (D/8)) + i, 16-byte column tid % (D/8)
  const int k_row0 = T::kKChunks * (tid / (D / 8));  // rows k_row0 + i: resource i starts i rows in
  const int k_col = tid % (D / 8);
  const uint32_t k_goff = (uint32_t)(k_row0 * D + k_col * 8) * 2;
  const int k_loff = k_row0 * T::kKPitch + k_col * 8;
  // V: rows 4*vg + jj, 16-byte column vc, written transposed
  const int vg = tid & 15;
  const int vc = tid >> 4;
  const bool v_task = T::kVTasks == kThreads || tid < T::kVTasks;
  const uint32_t v_goff = (uint32_t)(4 * vg * D + vc * 8) * 2;
  const int v_loff = vc * 8 * T::kVPitch + vt_pos(4 * vg);

  uint16_t* const kst[2] = {smem, smem + T::kKElems};
  uint16_t* const vst[2] = {smem + 2 * T::kKElems, smem + 2 * T::kKElems + T::kVElems};

  // tile r: position in the key sequence, valid rows, and segment row pointers
  struct TileLoc {
    int abs_base, rows;
    const uint16_t *k, *v;
  };
  auto locate = [&](int r) {
    const int t = t_begin + r;
    const bool own = t >= n_ct;
    const int local = (own ? t - n_ct : t) * kAttnBlockN;
    TileLoc L;
    L.abs_base = own ? a.len + local : local;
    L.rows = min(kAttnBlockN, (own ? self_rows : cache_rows) - local);
    L.k = (own ? ks_h : kc_h) + (int64_t)local * D;
    L.v = (own ? vs_h : vc_h) + (int64_t)local * D;
    return L;
  };
  // resource over rows [first, L.rows) of a tile, starting at row `first`
  auto row_rsrc = [&](const uint16_t* tile, int rows, int first) {
    const int n = max(rows - first, 0);
    return buffer_rsrc(tile + first * D, (uint32_t)n * D * 2);
  };
  u32x4 kreg[T::kKChunks];
  u32x4 vreg[4];
  auto load_k = [&](int r) {
    const TileLoc L = locate(r);
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) kreg[i] = buffer_load16(row_rsrc(L.k, L.rows, i), k_goff);
  };
  auto load_v = [&](int r) {
    const TileLoc L = locate(r);
    if (v_task) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) vreg[jj] = buffer_load16(row_rsrc(L.v, L.rows, jj), v_goff);
    }
  };
  auto store_k = [&](uint16_t* stage) {
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i)
      *reinterpret_cast<u32x4*>(stage + k_loff + i * T::kKPitch) = kreg[i];
  };
  auto store_v = [&](uint16_t* stage) {
    if (v_task) {
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        *reinterpret_cast<u32x2*>(stage + v_loff + (2 * wd) * T::kVPitch) =
            u32x2{lo_halves(vreg[0][wd], vreg[1][wd]), lo_halves(vreg[2][wd], vreg[3][wd])};
        *reinterpret_cast<u32x2*>(stage + v_loff + (2 * wd + 1) * T::kVPitch) =
            u32x2{hi_halves(vreg[0][wd], vreg[1][wd]), hi_halves(vreg[2][wd], vreg[3][wd])};
      }
    }
  };
  // S^T of one 64-key tile from an LDS K stage
  auto qk = [&](const uint16_t* kstage, f32x16 (&s)[2]) {
    const uint16_t* lk = kstage + lrow * T::kKPitch + 8 * half;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(lk + kb * 32 * T::kKPitch + ks * 16);
        s[kb] = mfma32x32x16(ka, qf[ks], s[kb]);
      }
  };

  // Tile r of the pipeline. On entry S^T of tile r is in s_cur, K of tile r+1
  // and V of tile r are in LDS, and the registers hold K of tile r+2 and V of
  // tile r+1 (loaded during tile r-1). The QK^T products of tile r+1 are
  // issued before tile r's softmax, so the matrix cores work on them while
  // the vector unit runs the softmax.
  // S^T accumulators of the current and the next tile; the two swap roles
  // every tile (the loop is unrolled by two), so they are never copied
  f32x16 s_a[2], s_b[2];
  auto do_tile = [&](int r, uint16_t* k_this, uint16_t* k_next, uint16_t* v_this,
                     uint16_t* v_next, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    __syncthreads();  // tile r-1 done everywhere: k_this and v_next are free
    if (r + 2 < n_t) store_k(k_this);
    if (r + 1 < n_t) store_v(v_next);
    if (r + 3 < n_t) load_k(r + 3);
    if (r + 2 < n_t) load_v(r + 2);
    if (!wave_active) return;
    // block-causal mask, and the missing rows of a partial tile (at most a
    // few tiles per split; kept out of the common path)
    const TileLoc L = locate(r);
    if (__builtin_expect(L.rows < kAttnBlockN || L.abs_base + kAttnBlockN > kmin, 0)) {
      __asm__ volatile("" ::: "memory");  // keep this block a real branch
      const int lim = min(L.rows, kend - L.abs_base);  // visible keys of this lane's row
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = kb * 32 + 8 * (rr >> 2) + 4 * half + (rr & 3);
          s_cur[kb][rr] = key < lim ? s_cur[kb][rr] : kNegInf;
        }
    }
    // online softmax (exp2 domain): row max and the (rare) rescale
    float mloc = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mloc = fmaxf(mloc, s_cur[kb][rr]);
    const float mt = half_swap_max(mloc) * a.scale_log2;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0, 0)) {
      __asm__ volatile("" ::: "memory");  // keep the rare rescale a real branch
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < T::kDBlocks; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    // S^T of tile r+1 on the matrix cores (on a stale stage after the last
    // tile; unused then) interleaved with tile r's exponentials on the VALU:
    // MFMA i = (key block i/kDSteps, d-step i%kDSteps) carries softmax
    // elements kPerMfma*i.. (block 0 of S(t+1) is accumulated while block 0
    // of S(t) is consumed, so block 1 of S(t+1) can reuse its registers) and
    // takes its K fragment from an LDS read issued two MFMAs earlier.
    constexpr int kQK = 2 * T::kDSteps;  // MFMAs of one S^T tile
    constexpr int kPerMfma = 32 / kQK;   // softmax elements per MFMA
    const uint16_t* lk = k_next + lrow * T::kKPitch + 8 * half;
    auto k_frag = [&](int i) {
      return *reinterpret_cast<const u32x4*>(lk + (i / T::kDSteps) * 32 * T::kKPitch +
                                             (i % T::kDSteps) * 16);
    };
    s_nxt[0] = f32x16{};
    s_nxt[1] = f32x16{};
    u32x4 pb[2][2];
    float pe[32];
    u32x4 kf[kQK];
    kf[0] = k_frag(0);
    kf[1] = k_frag(1);
#pragma unroll
    for (int i = 0; i < kQK; ++i) {
      if (i + 2 < kQK) kf[i + 2] = k_frag(i + 2);
      s_nxt[i / T::kDSteps] = mfma32x32x16(kf[i], qf[i % T::kDSteps], s_nxt[i / T::kDSteps]);
#pragma unroll
      for (int e = kPerMfma * i; e < kPerMfma * (i + 1); ++e)
        pe[e] = fast_exp2(__builtin_fmaf(s_cur[e >> 4][e & 15], a.scale_log2, -m_use));
#pragma unroll
      for (int e = kPerMfma * i; e < kPerMfma * (i + 1); e += 2) {
        const uint32_t w2 = pack_bf16x2(pe[e], pe[e + 1]);
        pb[e >> 4][(e >> 3) & 1][(e >> 1) & 3] = w2;
        l_run = add_bf16x2(w2, l_run);  // the denominator sums the rounded P
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // O^T += V^T P^T, V^T fragments read two MFMAs ahead
    constexpr int kPV = 4 * T::kDBlocks;
    const uint16_t* lv = v_this + lrow * T::kVPitch + 8 * half;
    auto v_frag = [&](int i) {  // i = (db, kb, ks2) with ks2 fastest
      return *reinterpret_cast<const u32x4*>(lv + (i >> 2) * 32 * T::kVPitch + ((i >> 1) & 1) * 32 +
                                             (i & 1) * 16);
    };
    u32x4 vf[kPV];
    vf[0] = v_frag(0);
    vf[1] = v_frag(1);
#pragma unroll
    for (int i = 0; i < kPV; ++i) {
      if (i + 2 < kPV) vf[i + 2] = v_frag(i + 2);
      o[i >> 2] = mfma32x32x16(vf[i], pb[(i >> 1) & 1][i & 1], o[i >> 2]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_t > 0) {
    // prologue: K and V of tile 0 and K of tile 1 into LDS, S^T of tile 0,
    // then the loads of K(2) and V(1) in flight
    load_k(0);
    load_v(0);
    store_k(kst[0]);
    store_v(vst[0]);
    if (n_t > 1) {
      load_k(1);
      store_k(kst[1]);
    }
    __syncthreads();
    qk(kst[0], s_a);
    if (n_t > 2) load_k(2);
    if (n_t > 1) load_v(1);
  }
  // two tiles per iteration so every stage is fixed at compile time
  for (int r = 0; r < n_t; r += 2) {
    do_tile(r, kst[0], kst[1], vst[0], vst[1], s_a, s_b);
    if (r + 1 < n_t) do_tile(r + 1, kst[1], kst[0], vst[1], vst[0], s_b, s_a);
  }

  // ---- epilogue
  if (!wave_active) return;
  const float l_tot = half_swap_sum(l_run);
  if (qrow >= a.n_q) return;
  const int64_t row_id = (int64_t)h * a.n_q + qrow;
  if (a.n_splits == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* op = a.out + row_id * D + 4 * half;
#pragma unroll
    for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<u32x2*>(op + db * 32 + 8 * g) =
            u32x2{pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                  pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
  } else {
    const int64_t prow = (int64_t)split * a.heads * a.n_q + row_id;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* op = a.part_o + prow * D + 4 * half;
#pragma unroll
    for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(op + db * 32 + 8 * g) =
            f32x4{o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv,
                  o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
    if (half == 0) a.part_lse[prow] = l_tot > 0.f ? m_run + log2f(l_tot) : kNegInf;
  }
}

// Combine split partials: out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M),
// M = max_s lse_s. Bound by HBM (4 * splits * (D + 1) bytes read and 2 * D
// written per row). D/4 threads per row, 16-byte reads.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse,
                                                         uint16_t* __restrict__ out,
                                                         int rows, int n_splits) {
  constexpr int kTpr = D / 4;
  constexpr int kRpb = 256 / kTpr;
  const int row = blockIdx.x * kRpb + threadIdx.x / kTpr;
  const int c = threadIdx.x % kTpr;
  if (row >= rows) return;
  float mx = kNegInf;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, part_lse[(int64_t)s * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const float lse = part_lse[(int64_t)s * rows + row];
    const float wgt = lse == kNegInf ? 0.f : fast_exp2(lse - mx);
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + ((int64_t)s * rows + row) * D + 4 * c);
    acc += wgt * v;
    wsum += wgt;
  }
  const float inv = 1.f / wsum;
  *reinterpret_cast<u32x2*>(out + (int64_t)row * D + 4 * c) =
      u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
}

}  // namespace

hipError_t launch_attn_partial(const AttnArgs& a, int head_dim, hipStream_t stream) {
  const unsigned grid = (unsigned)((a.n_items + 7) / 8 * 8);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_partial_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_partial_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const float* part_o, const float* part_lse, uint16_t* out,
                             int heads, int n_q, int head_dim, int n_splits,
                             hipStream_t stream) {
  const int rows = heads * n_q;
  const int rpb = 256 / (head_dim / 4);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(grid), dim3(256), 0, stream,
                       part_o, part_lse, out, rows, n_splits);
  else
    hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(grid), dim3(256), 0, stream,
                       part_o, part_lse, out, rows, n_splits);
  return hipGetLastError();
}

}  // namespace ws
