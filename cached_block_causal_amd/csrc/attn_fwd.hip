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
//  * K/V tiles of 64 keys are double-buffered in LDS (72 KB at D = 128, so two
//    workgroups fit in a CU's 160 KB) with the next tile's global loads in
//    flight during the current tile's MFMAs; one barrier per tile.
//  * Work items (head, split, query tile) are ordered with the query tile
//    fastest and mapped onto blockIdx so that the items of one (head, split)
//    land on the same XCD (workgroups are dispatched round-robin over the 8
//    XCDs): the K/V chunk they share is then served from that XCD's L2.
//  * Keys past a row's visible range read as zeros from global memory and are
//    masked to -inf, so unused cache capacity never reaches the arithmetic.
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

// Row j of the concatenated keys (cache rows, then own tokens); NULL past kmax.
__device__ __forceinline__ const uint16_t* key_row(const uint16_t* cache_h, const uint16_t* self_h,
                                                   int len, int kmax, int j, int d) {
  if (j >= kmax) return nullptr;
  return j < len ? cache_h + (int64_t)j * d : self_h + (int64_t)(j - len) * d;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_partial_kernel(const AttnArgs a) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::kStage];

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
  const int n_kt = (kmax + kAttnBlockN - 1) / kAttnBlockN;
  const int t_begin = (int)((int64_t)split * n_kt / a.n_splits);
  const int t_end = (int)((int64_t)(split + 1) * n_kt / a.n_splits);

  const uint16_t* kc_h = a.kc + h * a.cache_head_stride;
  const uint16_t* vc_h = a.vc + h * a.cache_head_stride;
  const uint16_t* ks_h = a.ks + (int64_t)h * a.n_self * D;
  const uint16_t* vs_h = a.vs + (int64_t)h * a.n_self * D;

  // ---- this lane's query row and its Q^T operands
  const int qrow = r0 + wave * 32 + lrow;
  const bool wave_active = r0 + wave * 32 < a.n_q;
  const int kend = qrow < a.n_q ? row_kend(a, qrow) : 0;
  u32x4 qf[T::kDSteps];
  {
    const uint16_t* qp = a.q + ((int64_t)h * a.n_q + qrow) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
      qf[ks] = qrow < a.n_q ? *reinterpret_cast<const u32x4*>(qp + ks * 16) : u32x4{0, 0, 0, 0};
  }

  f32x16 o[T::kDBlocks];
#pragma unroll
  for (int db = 0; db < T::kDBlocks; ++db) o[db] = f32x16{};
  float m_run = kNegInf;  // running max of scaled scores (log2 units)
  float l_run = 0.f;      // this lane's share of the softmax denominator

  // ---- global -> register staging of one tile
  u32x4 kreg[T::kKChunks];
  u32x4 vreg[4];
  const int vg = tid & 15;        // 4-key group of the V task
  const int vc = tid >> 4;        // 8-dim chunk of the V task
  auto load_tile = [&](int t) {
    const int base = t * kAttnBlockN;
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8), col = c % (D / 8);
      const uint16_t* p = key_row(kc_h, ks_h, a.len, kmax, base + row, D);
      kreg[i] = p ? *reinterpret_cast<const u32x4*>(p + col * 8) : u32x4{0, 0, 0, 0};
    }
    if (tid < T::kVTasks) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint16_t* p = key_row(vc_h, vs_h, a.len, kmax, base + 4 * vg + jj, D);
        vreg[jj] = p ? *reinterpret_cast<const u32x4*>(p + vc * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int st) {
    uint16_t* lk = smem + st * T::kStage;
    uint16_t* lv = lk + T::kKElems;
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8), col = c % (D / 8);
      *reinterpret_cast<u32x4*>(lk + row * T::kKPitch + col * 8) = kreg[i];
    }
    if (tid < T::kVTasks) {
      const int pos = vt_pos(4 * vg);
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const int d0 = vc * 8 + 2 * wd;
        *reinterpret_cast<u32x2*>(lv + d0 * T::kVPitch + pos) =
            u32x2{lo_halves(vreg[0][wd], vreg[1][wd]), lo_halves(vreg[2][wd], vreg[3][wd])};
        *reinterpret_cast<u32x2*>(lv + (d0 + 1) * T::kVPitch + pos) =
            u32x2{hi_halves(vreg[0][wd], vreg[1][wd]), hi_halves(vreg[2][wd], vreg[3][wd])};
      }
    }
  };

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
    __syncthreads();
  }

  for (int t = t_begin; t < t_end; ++t) {
    const int st = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    if (more) load_tile(t + 1);

    if (wave_active) {
      const uint16_t* lk = smem + st * T::kStage;
      const uint16_t* lv = lk + T::kKElems;
      // S^T for two 32-key blocks
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < T::kDSteps; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(
              lk + (kb * 32 + lrow) * T::kKPitch + ks * 16 + 8 * half);
          s[kb] = mfma32x32x16(ka, qf[ks], s[kb]);
        }
      }
      // block-causal mask and key-range tail
      const int base = t * kAttnBlockN;
      if (base + kAttnBlockN > kmin) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = base + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            s[kb][r] = key < kend ? s[kb][r] : kNegInf;
          }
      }
      // online softmax (exp2 domain)
      float mloc = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kb][r]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float mt = mloc * a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db) o[db] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      u32x4 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(__builtin_fmaf(s[kb][r], a.scale_log2, -m_use));
          l_run += p[r];
        }
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
          pb[kb][ks2] = u32x4{pack_bf16x2(p[8 * ks2 + 0], p[8 * ks2 + 1]),
                              pack_bf16x2(p[8 * ks2 + 2], p[8 * ks2 + 3]),
                              pack_bf16x2(p[8 * ks2 + 4], p[8 * ks2 + 5]),
                              pack_bf16x2(p[8 * ks2 + 6], p[8 * ks2 + 7])};
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ks2 = 0; ks2 < 2; ++ks2) {
            const u32x4 va = *reinterpret_cast<const u32x4*>(
                lv + (db * 32 + lrow) * T::kVPitch + kb * 32 + ks2 * 16 + 8 * half);
            o[db] = mfma32x32x16(va, pb[kb][ks2], o[db]);
          }
    }

    if (more) store_tile(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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
