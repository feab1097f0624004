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
//  * K and V tiles of 64 keys go from global memory straight into LDS (buffer
//    loads with the LDS-destination bit: no staging registers), in natural
//    row order. A row is cut into 64-byte column groups of four 16-byte
//    chunks; the chunk slot inside a group is XOR-swizzled with bits 2-3 of
//    the row, so the 32 rows one MFMA operand read touches spread over all
//    LDS banks. The V^T operand of the PV product comes from the LDS
//    transpose read ds_read_b64_tr_b16 (two per MFMA), which hands each lane
//    4 keys of one dimension.
//  * Online softmax in the exp2 domain, fp32, with the running max allowed to
//    lag the true max by up to 2^8 before O and l are rescaled (rescales are
//    rare once the max settles; the result is the same up to rounding). The
//    scale times log2 e is folded into Q once (rounded back to bf16) and
//    every S^T chain starts from the accumulator -max, so the MFMAs hand the
//    exponent arguments straight to v_exp_f32.
//  * Software pipeline over 64-key tiles: while the vector unit runs the
//    softmax of tile t, the matrix cores compute S^T of tile t+1 (their order
//    is fixed with scheduling barriers), then O^T += V^T P^T of tile t. K and
//    V each have two LDS stages (64 KB at D = 128, two workgroups per CU); the
//    loads of K(t+2) and V(t+1) are issued when tile t starts and awaited at
//    its end, one barrier per tile. A tile never straddles the cache and the
//    own tokens; its rows are read through a buffer resource built per tile
//    with scalar instructions whose range ends at the tile's last valid row,
//    so missing rows read as zeros.
//  * Work items (head, split, query tile) are ordered with the query tile
//    fastest and mapped onto blockIdx so that the items of one (head, split)
//    land on the same XCD (workgroups are dispatched round-robin over the 8
//    XCDs): the K/V chunk they share is then served from that XCD's L2. The
//    query tiles go last to first, so that in a call spanning many units
//    (a block triangle of work) the tiles with the most keys start first.
//    Tiles past a query tile's last visible key are never loaded, and the
//    mask is applied only to tiles that reach past its first row's keys.
//  * Rows past the visible range read as zeros and are masked to -inf, so
//    unused cache capacity never reaches the arithmetic.
//  * Calls with at most 32 queries (the handful of audio tokens of a unit)
//    run a narrow kernel instead: one wave per (head, split) over 32-key
//    tiles, with its own two LDS stages and no barrier. Such a call is bound
//    by the K/V stream; the narrow form spends 4x fewer MFMAs on empty query
//    rows and fills the chip with more, shorter streams, and it reads whole
//    cache lines with non-temporal loads (each K/V byte is read once).
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
  static constexpr int kGroups = D / 32;                  // 64-byte column groups per row
  static constexpr int kGroupBytes = kAttnBlockN * 64;    // one group of a 64-row tile
  static constexpr int kStageBytes = kGroups * kGroupBytes;
  static constexpr int kDSteps = D / 16;   // k-steps of the QK^T product
  static constexpr int kDBlocks = D / 32;  // 32-dim blocks of O^T
  static_assert(kGroups == 2 || kGroups == 4, "head_dim 64 or 128");
};

typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle of the narrow kernel's LDS tiles (128-byte half rows): the
// 16-byte chunk c of row R's half sits in slot c ^ swz(R), swz(R) = row bits
// 1, 2, 3 reversed. Any 8 rows of one parity then spread one chunk over all
// slots (the 16-lane passes of the K reads), and rows R and R + 2 land in
// opposite halves of the slots (the 32-lane passes of the transposing V
// reads): both read patterns are free of bank conflicts.
__device__ __forceinline__ int swz(int row) {
  return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Visible-key count of a query row from the unit table: the key end of the
// last unit that starts at or before the row. kTable: the table is in device
// memory (a binary search; its row begins increase strictly), else in the
// launch arguments. The two are separate kernel instances, so the common
// in-argument case carries no code for the other.
template <bool kTable>
__device__ __forceinline__ int row_kend(const AttnArgs& a, int row) {
  if constexpr (kTable) {
    int lo = 0, hi = a.n_units - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.unit_table[mid] <= row) lo = mid;
      else hi = mid - 1;
    }
    return a.unit_table[a.n_units + 1 + lo];
  }
  int u = 0;
  while (u + 1 < a.n_units && a.q_unit_begin[u + 1] <= row) ++u;
  return a.unit_kend[u];
}
// The same for every lane's own row (0 for rows past n_q); with the table in
// the arguments the loop index is uniform, so it is read with scalar loads.
template <bool kTable>
__device__ __forceinline__ int lane_kend(const AttnArgs& a, int qrow) {
  if (qrow >= a.n_q) return 0;
  if constexpr (kTable) return row_kend<true>(a, qrow);
  int kend = 0;
  for (int u = 0; u < a.n_units; ++u) kend = qrow >= a.q_unit_begin[u] ? a.unit_kend[u] : kend;
  return kend;
}

// Column group G (byte offset G*64 within each row, passed as the scalar
// offset: the row offset stays in voff, so a row past the range still reads
// zeros) of a tile's rows into LDS at dst: lane l writes dst + 16*l. The
// instruction's immediate offset is left at 0 because it also moves the LDS
// destination.
template <int G>
__device__ __forceinline__ void dma_group(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, G * 64, 0, 0);
}

// s_waitcnt operand that waits for vector memory counter <= n (0..63) only:
// vmcnt is split over bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8)
// are left at their maxima.
constexpr int vmcnt_only(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
// s_waitcnt operand that waits for lgkmcnt == 0 only
constexpr int kLgkmZero = 0xC07F;

__device__ __forceinline__ u32x4 lds_read16(const char* base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(base + byte_off);
}

// 4 bf16 of one dimension from 4 consecutive V rows (LDS transpose read)
__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int byte_off) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + byte_off));
  return __builtin_bit_cast(u32x2, r);
}

template <int D, bool kTable>
__global__ __launch_bounds__(kThreads, 2) void attn_partial_kernel(const AttnArgs a) {
  using T = Tile<D>;
  // separate objects per stage, so memory dependences between the in-flight
  // global->LDS loads and the reads of the other stages are visibly absent
  __shared__ __attribute__((aligned(16))) char k_st0[T::kStageBytes];
  __shared__ __attribute__((aligned(16))) char k_st1[T::kStageBytes];
  __shared__ __attribute__((aligned(16))) char v_st0[T::kStageBytes];
  __shared__ __attribute__((aligned(16))) char v_st1[T::kStageBytes];

  // ---- work item: XCD-aware decode of (head, split, query tile)
  const int per_xcd = gridDim.x >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= a.n_items) return;
  // query tiles in decreasing order: with several units in one call the
  // later tiles see more keys, so the longest items are dispatched first
  const int qt = a.n_qtiles - 1 - w % a.n_qtiles;
  const int hs = w / a.n_qtiles;
  const int split = hs % a.n_splits;
  const int h = hs / a.n_splits;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lrow = lane & 31;
  const int half = lane >> 5;

  const int r0 = qt * kAttnBlockM;
  const int r_last = min(r0 + kAttnBlockM, a.n_q) - 1;
  const int kmin = row_kend<kTable>(a, r0);     // smallest visible range in this tile
  const int kmax = row_kend<kTable>(a, r_last);  // largest (kend is non-decreasing)
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
  // the unit of a row is the last non-empty unit starting at or before it
  const int kend = lane_kend<kTable>(a, qrow);
  u32x4 qf[T::kDSteps];  // loaded after the first tiles' loads are issued

  f32x16 o[T::kDBlocks];
#pragma unroll
  for (int db = 0; db < T::kDBlocks; ++db) o[db] = f32x16{};
  float m_run = kNegInf;  // running max of scaled scores (log2 units)
  // Scores are produced already shifted by m_off (m_run once that is
  // finite, else 0): every S^T chain starts from the accumulator -m_off.
  float m_off = 0.f;
  f32x16 neg_off = f32x16{};
  float l_run = 0.f;      // this lane's share of the softmax denominator

  // ---- LDS layout: byte (G, row, slot) = G * kGroupBytes + row * 64 + slot * 16
  // holds 16-byte chunk 4*G + (slot ^ ((row >> 2) & 3)) of the row.
  // DMA: wave w moves rows 16w .. 16w+15; lane l writes row 16w + l/4, slot l%4.
  const uint32_t dma_off = (uint32_t)((16 * wave + (lane >> 2)) * D * 2 + (((lane & 3) ^ (lane >> 4)) * 16));
  // K operand of MFMA (kb, ks): row kb*32 + lrow, chunk 2*ks + half
  const int k_ofs[2] = {lrow * 64 + (((0 + half) ^ ((lrow >> 2) & 3)) * 16),
                        lrow * 64 + (((2 + half) ^ ((lrow >> 2) & 3)) * 16)};
  // V^T operand of MFMA (db, kb, ks2), read e (keys +8e): lane 16g + 4s + q
  // reads row kb*32 + 16*ks2 + 8e + 4*half + s, dims db*32 + 16*(g&1) + 4q ..
  const int v_s = (lane >> 2) & 3, v_q = lane & 3, v_g1 = (lane >> 4) & 1;
  const int v_u = 2 * v_g1 + (v_q >> 1);
  const int v_ofs[2] = {(4 * half + v_s) * 64 + ((v_u ^ (0 + half)) * 16) + 8 * (v_q & 1),
                        (4 * half + v_s) * 64 + ((v_u ^ (2 + half)) * 16) + 8 * (v_q & 1)};

  char* const kst[2] = {k_st0, k_st1};
  char* const vst[2] = {v_st0, v_st1};

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
    // tiles r >= n_t (past the split's end) are empty ranges: their loads
    // read zeros and move nothing, and their scores are masked entirely.
    // (The clamp would otherwise become a VALU med3, making the resource look
    // per-lane and every load a waterfall loop.)
    L.rows = __builtin_amdgcn_readfirstlane(
        r < n_t ? max(0, min(kAttnBlockN, (own ? self_rows : cache_rows) - local)) : 0);
    L.k = (own ? ks_h : kc_h) + (int64_t)local * D;
    L.v = (own ? vs_h : vc_h) + (int64_t)local * D;
    return L;
  };
  // this wave's share of a tile: rows 16w.. of every column group, into LDS
  auto dma_tile = [&](const uint16_t* rows_ptr, int rows, char* stage) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(rows_ptr, (uint32_t)rows * D * 2);
    char* dst = stage + wave * 1024;
    dma_group<0>(rs, dst, dma_off);
    dma_group<1>(rs, dst + T::kGroupBytes, dma_off);
    if constexpr (T::kGroups == 4) {
      dma_group<2>(rs, dst + 2 * T::kGroupBytes, dma_off);
      dma_group<3>(rs, dst + 3 * T::kGroupBytes, dma_off);
    }
  };
  auto dma_k = [&](int r, char* stage) {
    const TileLoc L = locate(r);
    dma_tile(L.k, L.rows, stage);
  };
  auto dma_v = [&](int r, char* stage) {
    const TileLoc L = locate(r);
    dma_tile(L.v, L.rows, stage);
  };
  auto k_frag = [&](const char* kstage, int kb, int ks) {
    return lds_read16(kstage, (ks >> 1) * T::kGroupBytes + kb * 32 * 64 + k_ofs[ks & 1]);
  };
  auto v_frag = [&](const char* vstage, int i) {  // i = (db, kb, ks2) with ks2 fastest
    const int db = i >> 2, kb = (i >> 1) & 1, ks2 = i & 1;
    const char* b = vstage + db * T::kGroupBytes + (kb * 32 + 16 * ks2) * 64;
    const u32x2 lo = lds_read_tr(b, v_ofs[0]);
    const u32x2 hi = lds_read_tr(b + 8 * 64, v_ofs[1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // S^T of one 64-key tile from an LDS K stage
  auto qk = [&](const char* kstage, f32x16 (&s)[2]) {
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma32x32x16(k_frag(kstage, kb, ks), qf[ks], ks == 0 ? neg_off : s[kb]);
  };
  // the tile's global loads into LDS are complete for this wave, then for all
  auto stage_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  };

  // block-causal mask and the missing rows of a partial tile r on its scores
  // (at most a few tiles per split): returns whether tile r needs it
  auto needs_mask = [&](int r) {
    const TileLoc L = locate(r);
    return L.rows < kAttnBlockN || L.abs_base + kAttnBlockN > kmin;
  };
  auto apply_mask = [&](int r, f32x16 (&sc)[2]) {
    const TileLoc L = locate(r);
    const int lim = min(L.rows, kend - L.abs_base);  // visible keys of this lane's row
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = kb * 32 + 8 * (rr >> 2) + 4 * half + (rr & 3);
        sc[kb][rr] = key < lim ? sc[kb][rr] : kNegInf;
      }
  };
  auto tile_max = [&](const f32x16 (&sc)[2]) {
    float m = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) m = fmaxf(m, sc[kb][rr]);
    return m;
  };
  // Fold a tile's local max (per lane, before the half-wave exchange, of the
  // shifted scores sc) into the running max. O and l are rescaled only when
  // the max grows by more than the slack, which is rare after the first
  // tiles; the offset then moves to the new max, sc with it.
  auto update_max = [&](f32x16 (&sc)[2], float mloc) {
    const float mt = half_swap_max(mloc) + m_off;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0, 0)) {
      __asm__ volatile("" ::: "memory");  // keep the rare rescale a real branch
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < T::kDBlocks; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      const float off_new = m_new == kNegInf ? 0.f : m_new;
      const float shift = m_off - off_new;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sc[kb] += shift;
      m_off = off_new;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) neg_off[rr] = -off_new;
    }
  };
  // mask (if needed) and max of tile r's scores, then the running max
  auto prepare = [&](int r, f32x16 (&sc)[2], float mloc) {
    if (__builtin_expect(needs_mask(r), 0)) {
      __asm__ volatile("" ::: "memory");  // keep this block a real branch
      apply_mask(r, sc);
      mloc = tile_max(sc);
    }
    update_max(sc, mloc);
  };

  // Tile r of the pipeline. On entry the masked S^T of tile r is in s_cur and
  // the running max covers it; K of tile r+1 and V of tile r are in LDS. The
  // loads of K(r+2) and V(r+1) go into the stages tile r-1 finished with.
  // Four blocks of 8 MFMAs keep the vector unit busy beside the matrix cores
  // (their order is fixed with scheduling barriers):
  //   1: S^T(r+1) key block 0   || exp of S(r) key block 0 -> P block 0
  //   2: O^T += V^T P, keys 0-31 || exp of S(r) key block 1 -> P block 1
  //   3: S^T(r+1) key block 1   || max over S(r+1) key block 0
  //   4: O^T += V^T P, keys 32-63 || max over S(r+1) key block 1 (second half)
  f32x16 s_a[2], s_b[2];
  auto do_tile = [&](int r, char* k_this, char* k_next, char* v_this, char* v_next,
                     f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    dma_k(r + 2, k_this);  // past the split's end: empty ranges, nothing read
    dma_v(r + 1, v_next);
    if (wave_active) {
      constexpr int kB = T::kDSteps;  // MFMAs per block (8 at D = 128)
      u32x4 pb[2][2];
      // Softmax of S(r) (scores already scaled and shifted), pipelined over
      // the 16 MFMA slots of blocks 1-2 (pair j = elements 2j, 2j+1 of the
      // lane's 32 scores): slot j exponentiates pair j and packs pair j-1 to
      // bf16 (adding it to the denominator), so no vector instruction of a
      // slot waits for another one of the same slot.
      float ex[32];
      auto exp_pair = [&](int j) {
        ex[2 * j] = fast_exp2(s_cur[j >> 3][(2 * j) & 15]);
        ex[2 * j + 1] = fast_exp2(s_cur[j >> 3][(2 * j + 1) & 15]);
      };
      auto pack_pair = [&](int j) {
        const uint32_t w2 = pack_bf16x2(ex[2 * j], ex[2 * j + 1]);
        pb[j >> 3][(j >> 2) & 1][j & 3] = w2;
        l_run = add_bf16x2(w2, l_run);  // the denominator sums the rounded P
      };
      // slot j's share; the empty asm keeps each result in its slot
      auto softmax_slot = [&](int j) {
        if (j < 16) exp_pair(j);
        if (j >= 1) pack_pair(j - 1);
        if (j < 16) __asm__ volatile("" : "+v"(ex[2 * j]), "+v"(ex[2 * j + 1]));
        __asm__ volatile("" : "+v"(l_run));
      };
      // S^T(r+1) key block kb, MFMA i of kB, K fragments two ahead
      u32x4 kf[2 * kB];
      auto qk_step = [&](int kb, int i) {
        if (i == 0) {
          kf[kb * kB + 0] = k_frag(k_next, kb, 0);
          kf[kb * kB + 1] = k_frag(k_next, kb, 1);
        }
        if (i + 2 < kB) kf[kb * kB + i + 2] = k_frag(k_next, kb, i + 2);
        s_nxt[kb] = mfma32x32x16(kf[kb * kB + i], qf[i], i == 0 ? neg_off : s_nxt[kb]);
      };
      // O^T += V^T P for key block kb, MFMA i of kB = (db, ks2), V^T two ahead
      u32x4 vf[2 * kB];
      auto pv_step = [&](int kb, int i) {
        auto frag = [&](int j) { return v_frag(v_this, (j >> 1) * 4 + kb * 2 + (j & 1)); };
        if (i == 0) {
          vf[kb * kB + 0] = frag(0);
          vf[kb * kB + 1] = frag(1);
        }
        if (i + 2 < kB) vf[kb * kB + i + 2] = frag(i + 2);
        o[i >> 1] = mfma32x32x16(vf[kb * kB + i], pb[kb][i & 1], o[i >> 1]);
      };
      constexpr int kEl = 16 / kB;  // max elements per MFMA in blocks 3-4
      constexpr int kPp = 8 / kB;   // softmax pairs per MFMA in blocks 1-2
#pragma unroll
      for (int i = 0; i < kB; ++i) {  // block 1
        qk_step(0, i);
#pragma unroll
        for (int j = kPp * i; j < kPp * (i + 1); ++j) softmax_slot(j);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < kB; ++i) {  // block 2
        pv_step(0, i);
#pragma unroll
        for (int j = 8 + kPp * i; j < 8 + kPp * (i + 1); ++j) softmax_slot(j);
        __builtin_amdgcn_sched_barrier(0);
      }
      float mloc = kNegInf;
#pragma unroll
      for (int i = 0; i < kB; ++i) {  // block 3
        qk_step(1, i);
        if (i == 0) softmax_slot(16);  // the last pack
#pragma unroll
        for (int rr = kEl * i; rr < kEl * (i + 1); ++rr) mloc = fmaxf(mloc, s_nxt[0][rr]);
        __asm__ volatile("" : "+v"(mloc));  // keep the max in this group
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < kB; ++i) {  // block 4; key block 1 of S(r+1) is read
        pv_step(1, i);                // once its MFMA chain has had time to finish
        if (i >= kB / 2) {
#pragma unroll
          for (int rr = 2 * kEl * (i - kB / 2); rr < 2 * kEl * (i - kB / 2 + 1); ++rr)
            mloc = fmaxf(mloc, s_nxt[1][rr]);
          __asm__ volatile("" : "+v"(mloc));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      prepare(r + 1, s_nxt, mloc);  // (after the last tile: scores unused)
    }
    stage_barrier();  // K(r+2), V(r+1) landed; tile r done everywhere
  };

  // prologue: K and V of tile 0 and K of tile 1 into LDS, then Q, so that
  // the first tiles and Q travel together
  if (n_t > 0) {
    dma_k(0, kst[0]);
    dma_v(0, vst[0]);
    dma_k(1, kst[1]);
  }
  {
    const uint16_t* qp = a.q + ((int64_t)h * a.n_q + qrow) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
      qf[ks] = qrow < a.n_q ? *reinterpret_cast<const u32x4*>(qp + ks * 16) : u32x4{0, 0, 0, 0};
    // wait for Q and the first tiles here, once: otherwise paths that skip
    // the prologue leave the loads pending and every tile's first MFMA would
    // wait on all loads
    __builtin_amdgcn_s_waitcnt(0);
    // fold the softmax scale (times log2 e) into Q, rounded back to bf16: the
    // MFMAs then produce scores in log2 units and the softmax needs no
    // multiply (one more bf16 rounding of each q element, within the
    // tolerance of the result)
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        qf[ks][w] = pack_bf16x2(bf16_lo(qf[ks][w]) * a.scale_log2, bf16_hi(qf[ks][w]) * a.scale_log2);
  }
  if (n_t > 0) {
    // S^T of tile 0 once every wave's share of the first tiles has landed
    __syncthreads();
    qk(kst[0], s_a);
    if (wave_active) prepare(0, s_a, tile_max(s_a));
    __syncthreads();  // every wave is done with K(0) before K(2) replaces it
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

// Narrow calls (all queries in one 32-row block, e.g. the 4 audio queries of
// a unit): the main kernel would keep three of its four waves idle, and the
// call is bound by HBM. Here one workgroup is one wave and one (head, split):
// it streams 32-key tiles of K and V through its own two LDS stages (16 KB
// each at D = 128) with no barrier, and per tile computes S^T (8 MFMAs at
// D = 128), the softmax of 16 scores per lane and O^T += V^T P^T (8 MFMAs).
// Partials go through the same workspace and merge as the main kernel's.
template <int D, bool kTable>
__global__ __launch_bounds__(64) void attn_narrow_kernel(const AttnArgs a) {
  using T = Tile<D>;
  constexpr int kN = kAttnNarrowN;            // keys per tile
  constexpr int kSB = kN * D * 2;             // one stage (a tile of K or V)
  constexpr int kLoads = kSB / 1024;          // 1 KB loads per tile and operand
  __shared__ __attribute__((aligned(16))) char k_st0[kSB];
  __shared__ __attribute__((aligned(16))) char k_st1[kSB];
  __shared__ __attribute__((aligned(16))) char v_st0[kSB];
  __shared__ __attribute__((aligned(16))) char v_st1[kSB];

  const int w = blockIdx.x;
  if (w >= a.n_items) return;
  const int split = w % a.n_splits;
  const int h = w / a.n_splits;
  const int lane = threadIdx.x;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  const int kmin = row_kend<kTable>(a, 0);
  const int kmax = row_kend<kTable>(a, a.n_q - 1);
  const int cache_rows = min(a.len, kmax);
  const int self_rows = max(0, kmax - a.len);
  const int n_ct = (cache_rows + kN - 1) / kN;
  const int n_kt = n_ct + (self_rows + kN - 1) / kN;
  const int t_begin = (int)((int64_t)split * n_kt / a.n_splits);
  const int n_t = (int)((int64_t)(split + 1) * n_kt / a.n_splits) - t_begin;

  const uint16_t* kc_h = a.kc + h * a.cache_head_stride;
  const uint16_t* vc_h = a.vc + h * a.cache_head_stride;
  const uint16_t* ks_h = a.ks + (int64_t)h * a.n_self * D;
  const uint16_t* vs_h = a.vs + (int64_t)h * a.n_self * D;

  const int qrow = lrow;
  const int kend = lane_kend<kTable>(a, qrow);
  u32x4 qf[T::kDSteps];
  {
    const uint16_t* qp = a.q + ((int64_t)h * a.n_q + qrow) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
      qf[ks] = qrow < a.n_q ? *reinterpret_cast<const u32x4*>(qp + ks * 16) : u32x4{0, 0, 0, 0};
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qf[ks][e] = pack_bf16x2(bf16_lo(qf[ks][e]) * a.scale_log2, bf16_hi(qf[ks][e]) * a.scale_log2);
  }
  f32x16 o[T::kDBlocks];
#pragma unroll
  for (int db = 0; db < T::kDBlocks; ++db) o[db] = f32x16{};
  float m_run = kNegInf, m_off = 0.f, l_run = 0.f;
  f32x16 neg_off = f32x16{};

  // LDS layout: byte (h, row, slot) = h*kHB + row*128 + slot*16 holds chunk
  // slot ^ swz(row) of the row's 128-byte half h (dims 64h + 8c ..). One load
  // moves 8 rows x 128 bytes, so each group of 8 lanes reads a whole cache
  // line, and the loads are non-temporal: every K/V byte of the call is read
  // once, and a stream of whole lines that does not stay in the L2 reaches
  // the memory's pace (half lines, or lines kept in the L2, do not).
  // Load b moves rows 8b .. 8b+7: lane l writes row 8b + l/8, slot l%8.
  constexpr int kHB = kN * 128;   // one half of a tile
  constexpr int kH = D / 64;      // halves per row
  const int dma_j = lane >> 3, dma_p = lane & 7;
  uint32_t dma_off[kN / 8];
#pragma unroll
  for (int b = 0; b < kN / 8; ++b)
    dma_off[b] = (uint32_t)((8 * b + dma_j) * D * 2 + ((dma_p ^ swz(8 * b + dma_j)) * 16));
  // K operand of MFMA ks: row lrow, dims 16ks + 8half ..: half ks/4, chunk
  // 2(ks%4) + half; one offset per ks%4
  int k_ofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) k_ofs[j] = lrow * 128 + (((2 * j + half) ^ swz(lrow)) * 16);
  // V^T operand of MFMA (db, ks2), read e (keys +8e): lane 16g + 4s + q reads
  // row 16*ks2 + 8e + 4*half + s, dims db*32 + 16*(g&1) + 4q .., i.e. half
  // db/2, chunk 4(db&1) + 2(g&1) + q/2, with swz(row) = 4(s/2) + 2half + e;
  // one offset per (db&1, e)
  const int v_s = (lane >> 2) & 3, v_q = lane & 3, v_g1 = (lane >> 4) & 1;
  const int v_u = 2 * v_g1 + (v_q >> 1);
  int v_ofs[2][2];
#pragma unroll
  for (int d1 = 0; d1 < 2; ++d1)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      v_ofs[d1][e] = (4 * half + v_s) * 128 + 16 * (4 * (d1 ^ (v_s >> 1)) + (v_u ^ (2 * half + e))) +
                     8 * (v_q & 1);

  struct TileLoc {
    int abs_base, rows;
    const uint16_t *k, *v;
  };
  auto locate = [&](int r) {  // r in [0, n_t + 2); r >= n_t is an empty tile
    const int t = t_begin + r;
    const bool own = t >= n_ct;
    const int local = (own ? t - n_ct : t) * kN;
    TileLoc L;
    L.abs_base = own ? a.len + local : local;
    L.rows = __builtin_amdgcn_readfirstlane(
        r < n_t ? max(0, min(kN, (own ? self_rows : cache_rows) - local)) : 0);
    L.k = (own ? ks_h : kc_h) + (int64_t)local * D;
    L.v = (own ? vs_h : vc_h) + (int64_t)local * D;
    return L;
  };
  auto dma_tile = [&](const uint16_t* rows_ptr, int rows, char* stage) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(rows_ptr, (uint32_t)rows * D * 2);
    // (the half's byte offset is the scalar offset, inside the row, so rows
    // past the range still read zeros; aux 2 = non-temporal)
#pragma unroll
    for (int b = 0; b < kN / 8; ++b)
#pragma unroll
      for (int h = 0; h < kH; ++h)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(stage + h * kHB + b * 1024), 16,
                                                 dma_off[b], h * 128, 0, 2);
  };
  auto dma = [&](int r, char* ks_stage, char* vs_stage) {
    const TileLoc L = locate(r);
    dma_tile(L.k, L.rows, ks_stage);
    dma_tile(L.v, L.rows, vs_stage);
  };

  auto tile = [&](int r, const char* kst, const char* vst) {
    // S^T of the tile's 32 keys (lane: query lrow, 16 keys)
    f32x16 sc = neg_off;
#pragma unroll
    for (int ks = 0; ks < T::kDSteps; ++ks)
      sc = mfma32x32x16(lds_read16(kst, (ks >> 2) * kHB + k_ofs[ks & 3]), qf[ks], sc);
    // mask the keys past the tile's rows or this row's visible range
    const TileLoc L = locate(r);
    if (__builtin_expect(L.rows < kN || L.abs_base + kN > kmin, 0)) {
      const int lim = min(L.rows, kend - L.abs_base);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = 8 * (rr >> 2) + 4 * half + (rr & 3);
        sc[rr] = key < lim ? sc[rr] : kNegInf;
      }
    }
    float mloc = kNegInf;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) mloc = fmaxf(mloc, sc[rr]);
    const float mt = half_swap_max(mloc) + m_off;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0, 0)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < T::kDBlocks; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      const float off_new = m_new == kNegInf ? 0.f : m_new;
      sc += m_off - off_new;
      m_off = off_new;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) neg_off[rr] = -off_new;
    }
    // P in bf16 (B operand of O^T += V^T P^T) and the denominator
    u32x4 pb[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w2 = pack_bf16x2(fast_exp2(sc[2 * j]), fast_exp2(sc[2 * j + 1]));
      pb[j >> 2][j & 3] = w2;
      l_run = add_bf16x2(w2, l_run);
    }
#pragma unroll
    for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const char* b = vst + (db >> 1) * kHB + 16 * ks2 * 128;
        const u32x2 lo = lds_read_tr(b, v_ofs[db & 1][0]);
        const u32x2 hi = lds_read_tr(b + 8 * 128, v_ofs[db & 1][1]);
        o[db] = mfma32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[ks2], o[db]);
      }
  };

  // Tile r reads stage r % 2 while the loads of tile r+1 fill the other one.
  // Only this wave touches its stages: before loads overwrite a stage, its
  // LDS reads (of tile r-1) must have returned (lgkmcnt 0); before a tile is
  // read, its own loads must have landed (vmcnt <= the next tile's loads).
  if (n_t > 0) dma(0, k_st0, v_st0);
  for (int r = 0; r < n_t; r += 2) {
    __builtin_amdgcn_s_waitcnt(kLgkmZero);
    __asm__ volatile("" ::: "memory");
    dma(r + 1, k_st1, v_st1);  // past the split's end: empty ranges, nothing read
    __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kLoads));
    __asm__ volatile("" ::: "memory");
    tile(r, k_st0, v_st0);
    if (r + 1 >= n_t) break;
    __builtin_amdgcn_s_waitcnt(kLgkmZero);
    __asm__ volatile("" ::: "memory");
    dma(r + 2, k_st0, v_st0);
    __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kLoads));
    __asm__ volatile("" ::: "memory");
    tile(r + 1, k_st1, v_st1);
  }
  // loads past the split's end may still be in flight: they must land before
  // the workgroup exits and its LDS is handed to another
  __builtin_amdgcn_s_waitcnt(0x0F70);

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
// written per row). D/4 threads per group, 16-byte reads. With G = 1 a group
// walks all splits of a row; with G > 1 (many splits, few rows, as in the
// audio path) G groups take every G-th split of one row and their partial
// sums (each relative to its own max) are combined through LDS, so a row's
// loads are spread over G times more threads instead of one serial chain.
template <int D, int G>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse,
                                                         uint16_t* __restrict__ out,
                                                         int rows, int n_splits) {
  constexpr int kTpr = D / 4;              // threads per group (4 dims each)
  constexpr int kRpb = 256 / (kTpr * G);   // rows per block
  const int row_in_block = threadIdx.x / (kTpr * G);
  const int g = (threadIdx.x / kTpr) % G;
  const int c = threadIdx.x % kTpr;
  const int row = blockIdx.x * kRpb + row_in_block;
  const bool live = row < rows;
  float mx = kNegInf;
  // (the split loops are unrolled so that several independent loads are in
  // flight per thread)
  if (live)
#pragma unroll 4
    for (int s = g; s < n_splits; s += G) mx = fmaxf(mx, part_lse[(int64_t)s * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (live)
#pragma unroll 4
    for (int s = g; s < n_splits; s += G) {
      const float lse = part_lse[(int64_t)s * rows + row];
      const float wgt = lse == kNegInf ? 0.f : fast_exp2(lse - mx);
      const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + ((int64_t)s * rows + row) * D + 4 * c);
      acc += wgt * v;
      wsum += wgt;
    }
  if constexpr (G > 1) {
    __shared__ f32x4 s_acc[kRpb][G][kTpr];
    __shared__ float s_m[kRpb][G], s_w[kRpb][G];
    s_acc[row_in_block][g][c] = acc;
    if (c == 0) {
      s_m[row_in_block][g] = mx;
      s_w[row_in_block][g] = wsum;
    }
    __syncthreads();
    if (g != 0 || !live) return;
    float m_all = kNegInf;
#pragma unroll
    for (int i = 0; i < G; ++i) m_all = fmaxf(m_all, s_m[row_in_block][i]);
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    wsum = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float mi = s_m[row_in_block][i];
      const float f = mi == kNegInf ? 0.f : fast_exp2(mi - m_all);
      acc += f * s_acc[row_in_block][i][c];
      wsum += f * s_w[row_in_block][i];
    }
  } else {
    if (!live) return;
  }
  const float inv = 1.f / wsum;
  *reinterpret_cast<u32x2*>(out + (int64_t)row * D + 4 * c) =
      u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
}

constexpr int kTableChunk = 896;  // ints per launch (3.6 KB of arguments)
struct TableChunk {
  int* dst;
  int n;
  int v[kTableChunk];
};
__global__ __launch_bounds__(256) void unit_table_kernel(const TableChunk c) {
  for (int i = threadIdx.x; i < c.n; i += 256) c.dst[i] = c.v[i];
}

}  // namespace

hipError_t launch_unit_table(int* dst, const int* vals, int n, hipStream_t stream) {
  for (int b = 0; b < n; b += kTableChunk) {
    TableChunk c;
    c.dst = dst + b;
    c.n = n - b < kTableChunk ? n - b : kTableChunk;
    for (int i = 0; i < c.n; ++i) c.v[i] = vals[b + i];
    hipLaunchKernelGGL(unit_table_kernel, dim3(1), dim3(256), 0, stream, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool kTable>
hipError_t launch_attn_partial_t(const AttnArgs& a, int head_dim, hipStream_t stream) {
  if (attn_narrow(a.n_q)) {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_narrow_kernel<128, kTable>), dim3(a.n_items), dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_narrow_kernel<64, kTable>), dim3(a.n_items), dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((a.n_items + 7) / 8 * 8);
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_partial_kernel<128, kTable>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_partial_kernel<64, kTable>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_partial(const AttnArgs& a, int head_dim, hipStream_t stream) {
  return a.unit_table ? launch_attn_partial_t<true>(a, head_dim, stream)
                      : launch_attn_partial_t<false>(a, head_dim, stream);
}

hipError_t launch_attn_merge(const float* part_o, const float* part_lse, uint16_t* out,
                             int heads, int n_q, int head_dim, int n_splits,
                             hipStream_t stream) {
  const int rows = heads * n_q;
  // many splits: spread each row over 8 groups of threads
  const int groups = n_splits >= 16 ? 8 : 1;
  const int rpb = 256 / (head_dim / 4 * groups);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (head_dim == 128) {
    if (groups > 1)
      hipLaunchKernelGGL((attn_merge_kernel<128, 8>), dim3(grid), dim3(256), 0, stream,
                         part_o, part_lse, out, rows, n_splits);
    else
      hipLaunchKernelGGL((attn_merge_kernel<128, 1>), dim3(grid), dim3(256), 0, stream,
                         part_o, part_lse, out, rows, n_splits);
  } else {
    if (groups > 1)
      hipLaunchKernelGGL((attn_merge_kernel<64, 8>), dim3(grid), dim3(256), 0, stream,
                         part_o, part_lse, out, rows, n_splits);
    else
      hipLaunchKernelGGL((attn_merge_kernel<64, 1>), dim3(grid), dim3(256), 0, stream,
                         part_o, part_lse, out, rows, n_splits);
  }
  return hipGetLastError();
}

}  // namespace ws
