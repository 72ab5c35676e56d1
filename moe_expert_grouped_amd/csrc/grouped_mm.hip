// Ragged per-expert grouped GEMM on gfx950 bf16 MFMA.
//
// Computes, for every expert e with s = m_indptr[e], t = m_indptr[e+1],
//   out[s:t] = a[s:t] @ b[e]^T
// (flashinfer.grouped_mm.grouped_mm_bf16, formula).  The expert boundaries are
// read on the device only: each workgroup scans m_indptr into LDS, turns it
// into per-expert counts of BM-row tiles, and walks a flat tile index through
// that table -- empty experts own no tile and no row is padded in memory
// (the device-walk backend's behaviour described on the same page).
//
// Two kernels, chosen from host sizes: grouped_mm_kernel (below) for groups
// averaging fewer than 192 rows, grouped_mm_big_kernel (further down, with
// its own notes) for larger ones; the big kernel also serves FC1, whose
// epilogue applies the SwiGLU activation.
//
// grouped_mm_kernel structure
//   * tile BM x BN, K step 64; WM x WN waves, each owning a (BM/WM) x (BN/WN)
//     sub-tile of 32x32 v_mfma_f32_32x32x16_bf16 blocks (fp32 accumulators);
//   * global -> registers -> LDS, one barrier per K step; P K steps of global
//     loads are in flight in registers (small-row groups are bound by
//     streaming b from HBM, so the loads run well ahead) while the LDS copy
//     of the current step feeds the MFMAs;
//   * LDS rows are 128 bytes (64 bf16); the 16-byte chunk c of row r is stored
//     at chunk c ^ ((r ^ (r >> 3)) & 7), so both the row-contiguous stores and
//     the MFMA fragment loads (32 rows, same chunk) spread over all banks;
//   * persistent grid: each workgroup loops over tiles; tile order is grouped
//     (GROUP_M m-tiles share each n-panel) and cut into 8 contiguous runs,
//     one per XCD (workgroup id % 8), which keeps the shared a/b panels in
//     that XCD's L2;
//   * rows past the expert's end are clamped on load and masked on store;
//     waves whose rows all lie past the end skip their MFMAs.
#include "common.hpp"

namespace mi {
namespace {

constexpr int GM_MAX_EXPERTS = 1024;
constexpr int GM_GROUP_M = 8;

// 16-byte chunk c of LDS row r sits at c ^ swz(r): consecutive rows spread over all banks
template <int CPR>  // chunks per row
__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row / CPR)) & (CPR - 1); }

template <int C>
__device__ __forceinline__ void gm_gload(u32x4 (&r)[C], const uint16_t* __restrict__ base,
                                         const long (&off)[C], int k0) {
#pragma unroll
  for (int i = 0; i < C; ++i) r[i] = *reinterpret_cast<const u32x4*>(base + off[i] + k0);
}

template <int C>
__device__ __forceinline__ void gm_lstore(uint16_t* lds, const u32x4 (&r)[C], const int (&off)[C]) {
#pragma unroll
  for (int i = 0; i < C; ++i) *reinterpret_cast<u32x4*>(lds + off[i]) = r[i];
}

// output element types: bf16 bits, fp16, fp32; one rounding to nearest even
struct Bf16Out { uint16_t bits; };
template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float v);
template <>
__device__ __forceinline__ void store_out<Bf16Out>(Bf16Out* p, float v) {
  p->bits = static_cast<uint16_t>(f32_to_bf16_rne(v));
}
template <>
__device__ __forceinline__ void store_out<_Float16>(_Float16* p, float v) {
  *p = static_cast<_Float16>(v);  // IEEE conversion, round to nearest even
}
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) {
  *p = v;
}

// the MFMA for the input type: bf16 or fp16 operands, fp32 accumulation
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int BM, int BN, int BK, int WM, int WN, int P, bool F16, typename OutT>
__global__ __launch_bounds__(64 * WM * WN) void grouped_mm_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ m_indptr, OutT* __restrict__ out, int m_rows, int k, int n,
    int E) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CPR = BK / 8;                // 16-byte chunks per LDS row
  constexpr int CPT_A = BM * BK / 8 / NT;  // 16-byte chunks per thread per stage
  constexpr int CPT_B = BN * BK / 8 / NT;
  constexpr int STAGE = (BM + BN) * BK;   // bf16 elements per stage
  static_assert(CPT_A * NT == BM * BK / 8 && CPT_B * NT == BN * BK / 8, "tile/threads");
  static_assert(FM >= 1 && FN >= 1, "wave tile");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  __shared__ int s_tile0[GM_MAX_EXPERTS + 1];  // first m-tile of each expert
  __shared__ int s_row0[GM_MAX_EXPERTS];       // clamped first row
  __shared__ int s_row1[GM_MAX_EXPERTS];       // clamped end row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- device-side walk of m_indptr: per-expert tile counts, prefix sum ----
  if (wave == 0) {
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        int s = min(max(m_indptr[e], 0), m_rows);
        int t = min(max(m_indptr[e + 1], s), m_rows);
        s_row0[e] = s;
        s_row1[e] = t;
        local += (t - s + BM - 1) / BM;
      }
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        s_tile0[e] = run;
        run += (s_row1[e] - s_row0[e] + BM - 1) / BM;
      }
    }
    if (lane == 63) s_tile0[E] = incl;
  }
  __syncthreads();

  const int total_mt = s_tile0[E];
  const int nt = n / BN;
  const long total = static_cast<long>(total_mt) * nt;
  // The dispatcher deals workgroup ids to the 8 XCDs in turn.  The tiles
  // (known only now) are cut into 8 contiguous runs, one per XCD, and the
  // workgroups of an XCD stride through its run.
  const int slots = gridDim.x >> 3;  // workgroups per XCD (grid is a multiple of 8)
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const long run = (total + 7) / 8;
  const long run_end = min(total, (xcd + 1) * run);

  uint16_t* const ldsA0 = smem;
  uint16_t* const ldsB0 = smem + BM * BK;

  for (long L = xcd * run + slot; L < run_end; L += slots) {

    // grouped order: GROUP_M consecutive m-tiles sweep each n-panel together
    const long span = static_cast<long>(GM_GROUP_M) * nt;
    const int grp = static_cast<int>(L / span);
    const int first = grp * GM_GROUP_M;
    const int gsize = min(total_mt - first, GM_GROUP_M);
    const int in_grp = static_cast<int>(L - static_cast<long>(grp) * span);
    const int gm = first + in_grp % gsize;
    const int ni = in_grp / gsize;

    // expert owning global m-tile gm: last e with s_tile0[e] <= gm
    int lo = 0, hi = E;  // s_tile0[lo] <= gm < s_tile0[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_tile0[mid] <= gm) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int m0 = s_row0[e] + (gm - s_tile0[e]) * BM;
    const int m_end = s_row1[e];
    const int n0 = ni * BN;

    const uint16_t* __restrict__ Ag = a;
    const uint16_t* __restrict__ Bg = b + (static_cast<long>(e) * n + n0) * k;

    // per-thread global chunk coordinates (fixed over the K loop)
    long a_off[CPT_A];
    int a_lds[CPT_A];
#pragma unroll
    for (int i = 0; i < CPT_A; ++i) {
      const int c = tid + i * NT;
      const int r = c / CPR, kc = c % CPR;
      const int gr = min(m0 + r, m_end - 1);
      a_off[i] = static_cast<long>(gr) * k + kc * 8;
      a_lds[i] = r * BK + ((kc ^ lds_swz<CPR>(r)) << 3);
    }
    long b_off[CPT_B];
    int b_lds[CPT_B];
#pragma unroll
    for (int i = 0; i < CPT_B; ++i) {
      const int c = tid + i * NT;
      const int r = c / CPR, kc = c % CPR;
      b_off[i] = static_cast<long>(r) * k + kc * 8;
      b_lds[i] = r * BK + ((kc ^ lds_swz<CPR>(r)) << 3);
    }

    const bool wave_active = (m0 + wm * WTM) < m_end;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    const int KT = k / BK;
    // P stages of global loads in flight in registers (indices clamped to the
    // last stage so every step issues the same loads); LDS double-buffered.
    u32x4 ra[P][CPT_A], rb[P][CPT_B];
    __syncthreads();  // previous tile's last LDS reads are done
#pragma unroll
    for (int q = 0; q < P; ++q) {
      gm_gload(ra[q], Ag, a_off, min(q, KT - 1) * BK);
      gm_gload(rb[q], Bg, b_off, min(q, KT - 1) * BK);
    }
    gm_lstore(ldsA0, ra[0], a_lds);
    gm_lstore(ldsB0, rb[0], b_lds);
    gm_gload(ra[0], Ag, a_off, min(P, KT - 1) * BK);
    gm_gload(rb[0], Bg, b_off, min(P, KT - 1) * BK);
    __syncthreads();

    for (int kt0 = 0; kt0 < KT; kt0 += P) {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int kt = kt0 + q;
        const int cur = kt & 1;
        {
          // steps past the end only refill and copy (no MFMAs): every step
          // issues the same loads
          if (wave_active && kt < KT) {
            const uint16_t* sA = ldsA0 + cur * STAGE;
            const uint16_t* sB = ldsB0 + cur * STAGE;
#pragma unroll
            for (int s = 0; s < BK / 16; ++s) {
              const int kc = 2 * s + (lane >> 5);
              u32x4 fa[FM], fb[FN];
#pragma unroll
              for (int i = 0; i < FM; ++i) {
                const int r = wm * WTM + i * 32 + (lane & 31);
                fa[i] = *reinterpret_cast<const u32x4*>(sA + r * BK + ((kc ^ lds_swz<CPR>(r)) << 3));
              }
#pragma unroll
              for (int j = 0; j < FN; ++j) {
                const int r = wn * WTN + j * 32 + (lane & 31);
                fb[j] = *reinterpret_cast<const u32x4*>(sB + r * BK + ((kc ^ lds_swz<CPR>(r)) << 3));
              }
#pragma unroll
              for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<F16>(fa[i], fb[j], acc[i][j]);
            }
          }
          // stage kt+1 sits in register slot (q+1) % P; refill that slot with stage kt+1+P
          const int nq = (q + 1) % P;
          gm_lstore(ldsA0 + (cur ^ 1) * STAGE, ra[nq], a_lds);
          gm_lstore(ldsB0 + (cur ^ 1) * STAGE, rb[nq], b_lds);
          gm_gload(ra[nq], Ag, a_off, min(kt + 1 + P, KT - 1) * BK);
          gm_gload(rb[nq], Bg, b_off, min(kt + 1 + P, KT - 1) * BK);
          __syncthreads();
        }
      }
    }

    // ---- epilogue: C[row][col], row = 8*(q/4) + 4*(lane/32) + q%4, col = lane%32 ----
    if (wave_active) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = m0 + wm * WTM + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
          if (row < m_end) {
            OutT* orow = out + static_cast<long>(row) * n + n0 + wn * WTN + (lane & 31);
#pragma unroll
            for (int j = 0; j < FN; ++j) store_out<OutT>(orow + j * 32, acc[i][j][q]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large groups: 256-column tiles of 256 or 128 rows, four wavefronts of 128
// rows each (one per SIMD), one tile per workgroup.
//
// Tiles.  Every expert's rows are cut into 256-row tiles; a last piece of at
// most 128 rows becomes a 128-row tile instead, which takes about half the
// time (at most 127 padded rows per expert instead of 255).  The 256-row tiles
// come first in the walk and the 128-row ones after; each list, in grouped
// order (GM_GROUP_M m-tiles sweep each n-panel together), is cut into 8
// contiguous runs, one per XCD, so the XCDs get equal work and each keeps its
// a and b panels in its own L2.
//
// K loop.  Per 64-wide K step every wavefront runs 4 sub-steps of
// v_mfma_f32_32x32x16 blocks (4 x FN of them).  The fragments of sub-step s+1
// are read from LDS while the MFMAs of sub-step s run (two fragment register
// sets), so with one wavefront per SIMD the LDS latency stays hidden.  The K
// step's one barrier sits before the last sub-step's MFMAs, and the next
// stage's first fragments are read right after it, under those MFMAs.  Global
// loads run GB_P K steps ahead in registers; the next stage is copied to the
// other LDS buffer during sub-step 1.  LDS rows are padded to 72 elements
// (144 bytes): the 32 rows of a fragment read and the 8 chunks of a row write
// both spread over all banks.
// ---------------------------------------------------------------------------
constexpr int GB_BN = 256, GB_BK = 64, GB_P = 2;
constexpr int GB_RS = GB_BK + 8;                 // padded LDS row (16-bit elements)
constexpr int GB_STAGE = (256 + GB_BN) * GB_RS;  // elements per LDS stage (largest tile)

// Device-side walk of m_indptr by wavefront 0: the clamped first row of every
// expert (s_row0[E] = the end of the last one), the first 256-row tile
// (s_full0) and the first 128-row tile (s_half0) of each expert.
__device__ __forceinline__ void gb_walk(const int32_t* __restrict__ m_indptr, int m_rows, int E,
                                        int* s_full0, int* s_half0, int* s_row0) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int nf = 0, nh = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int s = min(max(m_indptr[e], 0), m_rows);
      const int t = min(max(m_indptr[e + 1], s), m_rows);
      s_row0[e] = s;
      const int q = (t - s) >> 8, r = (t - s) & 255;
      nf += q + (r > 128);
      nh += (r > 0 && r <= 128);
    }
  }
  int incl_f = nf, incl_h = nh;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int vf = __shfl_up(incl_f, off, 64), vh = __shfl_up(incl_h, off, 64);
    if (lane >= off) {
      incl_f += vf;
      incl_h += vh;
    }
  }
  int run_f = incl_f - nf, run_h = incl_h - nh;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      s_full0[e] = run_f;
      s_half0[e] = run_h;
      const int s = s_row0[e];
      const int t = min(max(m_indptr[e + 1], s), m_rows);
      const int q = (t - s) >> 8, r = (t - s) & 255;
      run_f += q + (r > 128);
      run_h += (r > 0 && r <= 128);
    }
  }
  if (lane == 63) {
    s_full0[E] = incl_f;
    s_half0[E] = incl_h;
    s_row0[E] = min(max(m_indptr[E], 0), m_rows);
  }
}

// m-tile and n-panel of linear index L in the grouped order of a list of
// `count` m-tiles
__device__ __forceinline__ void gb_order(long L, int count, int nt, int& mt, int& ni) {
  const long span = static_cast<long>(GM_GROUP_M) * nt;
  const int grp = static_cast<int>(L / span);
  const int first = grp * GM_GROUP_M;
  const int gsize = min(count - first, GM_GROUP_M);
  const int in_grp = static_cast<int>(L - static_cast<long>(grp) * span);
  mt = first + in_grp % gsize;
  ni = in_grp / gsize;
}

// expert owning list entry mt: last e with pre[e] <= mt (pre non-decreasing,
// pre[0] = 0 <= mt < pre[E])
__device__ __forceinline__ int gb_owner(const int* pre, int E, int mt) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// four consecutive output columns of one row: one buffer store at byte offset
// `off`; a store past the descriptor's range is dropped
template <typename OutT>
__device__ __forceinline__ void bstore_out4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v);
template <>
__device__ __forceinline__ void bstore_out4<Bf16Out>(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                     f32x4 v) {
  typedef __bf16 b4 __attribute__((ext_vector_type(4)));
  // hardware conversion: round to nearest even
  const b4 h = __builtin_convertvector(v, b4);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, off, 0, 0);
}
template <>
__device__ __forceinline__ void bstore_out4<_Float16>(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                      f32x4 v) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 h = __builtin_convertvector(v, h4);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, off, 0, 0);
}
template <>
__device__ __forceinline__ void bstore_out4<float>(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

// Instruction interleave of a sub-step: the NR LDS reads of the next
// fragments go out between the first NR of its NM MFMAs, so they complete
// under this sub-step.
template <int NR, int NM>
__device__ __forceinline__ void gb_interleave_reads() {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
}
// sub-step 1 also copies the next stage to LDS (NC writes) and refills its
// register slot (NC global loads), spread over the remaining MFMAs
template <int NR, int NM, int NC>
__device__ __forceinline__ void gb_interleave_copy() {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
  constexpr int REST = NM - NR, PER = (NC + REST - 1) / REST;
#pragma unroll
  for (int i = 0; i < REST; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x200, PER, 0);  // LDS write
    __builtin_amdgcn_sched_group_barrier(0x020, PER, 0);  // global load
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
  }
}

// FC1 epilogue parameters: the gate/up halves of b and the SwiGLU activation
struct GbGlu {
  const uint16_t* delta;  // bf16 [m_rows, 2I] added before the activation, or null
  const float* alpha;     // [E] or null (1)
  const float* beta;      // [E] or null (0)
  const float* limit;     // [E] or null (no clamp)
};

// One output tile: 256 rows (FN = 4: waves 2 x 2, 128 x 128 each) or 128 rows
// (FN = 2: waves 1 x 4, 128 x 64 each), 256 columns.  `rows` (1..BM) of the
// tile belong to the expert; the a descriptor covers only those, so rows past
// them read as zero and their stores are dropped.
//
// GLU (FC1): b[e] is [n = 2I, k], gate rows 0..I-1 and up rows I..2I-1.  A
// tile then covers 128 output columns c0 = n0/2 ..: each wavefront's b
// fragments j < FN/2 are gate rows and j >= FN/2 the matching up rows, so one
// lane holds both operands of every output it writes; out is [m_rows, I].
template <int FN, bool F16, bool GLU, typename OutT>
__device__ __forceinline__ void gb_tile(const uint16_t* __restrict__ a,
                                        const uint16_t* __restrict__ b, OutT* __restrict__ out,
                                        uint16_t* smem, int e, int m0, int rows, int n0, int k,
                                        int n, const GbGlu& gl) {
  constexpr int WN = FN == 4 ? 2 : 4;        // wavefronts along n
  constexpr int BM = 128 * (4 / WN);         // tile rows
  constexpr int CPT_A = BM / 32, CPT_B = 8;  // 16-byte chunks per thread per stage
  constexpr int NR = 4 + FN, NM = 4 * FN;    // fragment reads and MFMAs per sub-step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, h = lane >> 5;
  const int KT = k / GB_BK;
  const uint32_t kbytes = static_cast<uint32_t>(k) * 2;

  const __amdgpu_buffer_rsrc_t ar = buf_rsrc(a + static_cast<long>(m0) * k, rows * kbytes);
  const int inter = n / 2, c0 = n0 / 2;  // GLU: output width and first output column
  const long b_row0 = static_cast<long>(e) * n + (GLU ? c0 : n0);
  const __amdgpu_buffer_rsrc_t br = buf_rsrc(
      b + b_row0 * k, static_cast<uint32_t>(GLU ? inter + 128 : GB_BN) * kbytes);
  // b row (relative to b_row0) of staging block i (LDS rows 32i .. 32i+31)
  uint32_t b_so[CPT_B];
#pragma unroll
  for (int i = 0; i < CPT_B; ++i) {
    int row = 32 * i;
    if constexpr (GLU) {
      const int jj = i % FN;  // fragment of wavefront i / FN
      row = (jj < FN / 2 ? 0 : inter) + (i / FN) * 16 * FN + (jj % (FN / 2)) * 32;
    }
    b_so[i] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(row) * kbytes);
  }

  // staging: chunk c = tid + 256 i is row c/8 = tid/8 + 32 i, 16-byte chunk
  // tid%8 of the stage
  const uint32_t g_off = static_cast<uint32_t>(tid >> 3) * kbytes + (tid & 7) * 16;
  const uint32_t g_step = 32 * kbytes;  // 32 rows
  const int st_lds = (tid >> 3) * GB_RS + (tid & 7) * 8;
  // fragments: lane (r, h) reads row r of each 32-row block, 16-byte chunk 2s+h
  const int fa_base = (wm * 128 + r) * GB_RS + 8 * h;
  const int fb_base = 256 * GB_RS + (wn * 32 * FN + r) * GB_RS + 8 * h;

  f32x16 acc[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  struct Frag {
    u32x4 a[4], b[FN];
  };
  u32x4 ra[GB_P][CPT_A], rb[GB_P][CPT_B];
  auto gload = [&](int p, int kt) {
    // stages past the end reload the last one: every step issues the same loads
    const uint32_t so = static_cast<uint32_t>(min(kt, KT - 1)) * (GB_BK * 2);
#pragma unroll
    for (int i = 0; i < CPT_A; ++i) ra[p][i] = buf_ld128(ar, g_off + i * g_step, so);
#pragma unroll
    for (int i = 0; i < CPT_B; ++i) rb[p][i] = buf_ld128(br, g_off, so + b_so[i]);
  };
  auto lstore = [&](int p, uint16_t* st) {
#pragma unroll
    for (int i = 0; i < CPT_A; ++i)
      *reinterpret_cast<u32x4*>(st + st_lds + i * 32 * GB_RS) = ra[p][i];
#pragma unroll
    for (int i = 0; i < CPT_B; ++i)
      *reinterpret_cast<u32x4*>(st + 256 * GB_RS + st_lds + i * 32 * GB_RS) = rb[p][i];
  };
  auto fload = [&](Frag& f, const uint16_t* st, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = *reinterpret_cast<const u32x4*>(st + fa_base + i * 32 * GB_RS + 16 * s);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      f.b[j] = *reinterpret_cast<const u32x4*>(st + fb_base + j * 32 * GB_RS + 16 * s);
  };
  // C[m][n] with m = output column (b row), n = output row (a row)
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<F16>(f.b[j], f.a[i], acc[i][j]);
  };

  Frag f0, f1;
#pragma unroll
  for (int p = 0; p < GB_P; ++p) {
    gload(p, p);
    __builtin_amdgcn_sched_barrier(0);  // slots in order: the loop's waits stay exact
  }
  lstore(0, smem);
  gload(0, GB_P);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  fload(f0, smem, 0);

  // one K step; `q` = register slot holding stage kt+1
  auto kstep = [&](int kt, int q) {
    uint16_t* st = smem + (kt & 1) * GB_STAGE;
    uint16_t* nx = smem + ((kt & 1) ^ 1) * GB_STAGE;
    fload(f1, st, 1);
    mma(f0);
    gb_interleave_reads<NR, NM>();
    __builtin_amdgcn_sched_barrier(0);
    fload(f0, st, 2);
    lstore(q, nx);
    gload(q, kt + 1 + GB_P);
    mma(f1);
    gb_interleave_copy<NR, NM, CPT_A + CPT_B>();
    __builtin_amdgcn_sched_barrier(0);
    fload(f1, st, 3);
    mma(f0);
    gb_interleave_reads<NR, NM>();
    __builtin_amdgcn_sched_barrier(0);
    // every wavefront's LDS work of this step is done: the next stage is
    // complete and this one may be overwritten one step later
    __syncthreads();
    fload(f0, nx, 0);
    mma(f1);
    gb_interleave_reads<NR, NM>();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The loop body is straight-line code (all MFMAs unconditional: rows past
  // the group's end are zeros), so the compiler's wait counts stay exact.
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    kstep(kt, 1);
    kstep(kt + 1, 0);
  }
  if (kt < KT) kstep(kt, 1);

  if (wm * 128 >= rows) return;  // all of this wavefront's rows lie past the group's end
  if constexpr (!GLU) {
    // acc[i][j][q]: tile row wm*128 + i*32 + r, column wn*32*FN + j*32 + 8*(q/4) + 4h + q%4.
    const __amdgpu_buffer_rsrc_t orsrc = buf_rsrc(out + static_cast<long>(m0) * n,
                                                  static_cast<uint32_t>(rows) * n * sizeof(OutT));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t orow =
          (static_cast<uint32_t>(wm * 128 + i * 32 + r) * n + n0 + wn * 32 * FN + 4 * h) *
          sizeof(OutT);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                           acc[i][j][4 * g + 3]};
          bstore_out4<OutT>(orsrc, orow + (j * 32 + 8 * g) * sizeof(OutT), v);
        }
      }
    }
  } else {
    // gate acc[i][j], up acc[i][j + FN/2] (j < FN/2): tile row wm*128 + i*32 + r,
    // output column c0 + wn*16*FN + j*32 + 8*(q/4) + 4h + q%4
    const float alpha = gl.alpha ? gl.alpha[e] : 1.f;
    const float beta = gl.beta ? gl.beta[e] : 0.f;
    const float limit = gl.limit ? gl.limit[e] : __builtin_inff();
    const __amdgpu_buffer_rsrc_t orsrc = buf_rsrc(
        out + static_cast<long>(m0) * inter, static_cast<uint32_t>(rows) * inter * sizeof(OutT));
    const bool has_delta = gl.delta != nullptr;
    const __amdgpu_buffer_rsrc_t drsrc =
        buf_rsrc(has_delta ? gl.delta + static_cast<long>(m0) * n : gl.delta,
                 has_delta ? static_cast<uint32_t>(rows) * n * 2 : 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t trow = wm * 128 + i * 32 + r;
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t col = c0 + wn * 16 * FN + j * 32 + 8 * g + 4 * h;
          float hg[4], hu[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            hg[q] = acc[i][j][4 * g + q];
            hu[q] = acc[i][j + FN / 2][4 * g + q];
          }
          if (has_delta) {
            const u32x2 dg = buf_ld64(drsrc, (trow * n + col) * 2, 0);
            const u32x2 du = buf_ld64(drsrc, (trow * n + inter + col) * 2, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t wg = dg[q >> 1], wu = du[q >> 1];
              hg[q] += __uint_as_float((q & 1) ? (wg & 0xffff0000u) : (wg << 16));
              hu[q] += __uint_as_float((q & 1) ? (wu & 0xffff0000u) : (wu << 16));
            }
          }
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gg = fminf(hg[q], limit);
            const float uu = fminf(fmaxf(hu[q], -limit), limit);
            // logistic function from the hardware exp2 and reciprocal (a few ulp)
            const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-alpha * gg));
            v[q] = gg * sig * (uu + beta);
          }
          bstore_out4<OutT>(orsrc, (trow * inter + col) * sizeof(OutT), v);
        }
      }
    }
  }
}

template <bool F16, bool GLU, typename OutT>
__global__ __launch_bounds__(256, 1) void grouped_mm_big_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ m_indptr, OutT* __restrict__ out, int m_rows, int k, int n,
    int E, GbGlu gl) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * GB_STAGE];
  __shared__ int s_full0[GM_MAX_EXPERTS + 1];
  __shared__ int s_half0[GM_MAX_EXPERTS + 1];
  __shared__ int s_row0[GM_MAX_EXPERTS + 1];

  if ((threadIdx.x >> 6) == 0) gb_walk(m_indptr, m_rows, E, s_full0, s_half0, s_row0);
  __syncthreads();

  const int nt = n / GB_BN;
  const int count_f = s_full0[E], count_h = s_half0[E];
  const long total_f = static_cast<long>(count_f) * nt, total_h = static_cast<long>(count_h) * nt;
  // The grid is an upper bound on the tiles; the dispatcher deals workgroup
  // ids to the 8 XCDs in turn.  An XCD's first run_f workgroups take its run
  // of the 256-row tiles, the next run_h its run of the 128-row tiles.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const long run_f = (total_f + 7) / 8, run_h = (total_h + 7) / 8;
  if (slot < run_f) {
    const long L = xcd * run_f + slot;
    if (L >= total_f) return;
    int mt, ni;
    gb_order(L, count_f, nt, mt, ni);
    const int e = __builtin_amdgcn_readfirstlane(gb_owner(s_full0, E, mt));
    const int m0 = __builtin_amdgcn_readfirstlane(s_row0[e] + (mt - s_full0[e]) * 256);
    const int end = max(s_row0[e + 1], s_row0[e]);
    const int rows = __builtin_amdgcn_readfirstlane(min(end - m0, 256));
    gb_tile<4, F16, GLU, OutT>(a, b, out, smem, e, m0, rows, ni * GB_BN, k, n, gl);
  } else {
    const long L = xcd * run_h + (slot - run_f);
    if (slot - run_f >= run_h || L >= total_h) return;
    int mt, ni;
    gb_order(L, count_h, nt, mt, ni);
    const int e = __builtin_amdgcn_readfirstlane(gb_owner(s_half0, E, mt));
    // the expert's last piece: after its 256-row tiles
    const int m0 = __builtin_amdgcn_readfirstlane(s_row0[e] + (s_full0[e + 1] - s_full0[e]) * 256);
    const int end = max(s_row0[e + 1], s_row0[e]);
    const int rows = __builtin_amdgcn_readfirstlane(end - m0);
    gb_tile<2, F16, GLU, OutT>(a, b, out, smem, e, m0, rows, ni * GB_BN, k, n, gl);
  }
}

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

template <int BM, int BN, int BK, int WM, int WN, int P, bool F16, typename OutT>
mi_status launch_grouped(const void* a, int64_t m_rows, int64_t k, const void* b,
                         int64_t batch, int64_t n, const int32_t* m_indptr, void* out,
                         hipStream_t stream, int occupancy) {
  const long ub_mtiles = (m_rows + BM - 1) / BM + batch;
  const long ub_tiles = ub_mtiles * (n / BN);
  long G = static_cast<long>(num_cus()) * occupancy;
  if (G > ub_tiles) G = ub_tiles;
  G = ((G + 7) / 8) * 8;
  if (G < 8) G = 8;
  hipLaunchKernelGGL((grouped_mm_kernel<BM, BN, BK, WM, WN, P, F16, OutT>), dim3(G), dim3(64 * WM * WN), 0,
                     stream, static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b),
                     m_indptr, static_cast<OutT*>(out), static_cast<int>(m_rows),
                     static_cast<int>(k), static_cast<int>(n), static_cast<int>(batch));
  return launch_status("grouped_mm_bf16");
}

template <bool F16, bool GLU, typename OutT>
mi_status launch_grouped_big(const void* a, int64_t m_rows, int64_t k, const void* b, int64_t batch,
                             int64_t n, const int32_t* m_indptr, void* out, hipStream_t stream,
                             const GbGlu& gl) {
  // one workgroup per tile of the upper bound (the real count is known on the
  // device only); each XCD's run of the real tiles fits in its G/8 ids
  const long ub_tiles = ((m_rows + 255) / 256 + batch) * (n / GB_BN);
  const long G = ((ub_tiles + 7) / 8 + 2) * 8;
  MI_REQUIRE(G < (1L << 31), "grouped_mm_bf16: problem too large");
  MI_REQUIRE(static_cast<uint64_t>(k) * 2 * (GLU ? n / 2 + 128 : GB_BN) < (1ULL << 32) &&
                 static_cast<uint64_t>(n) * 256 * sizeof(OutT) < (1ULL << 32),
             "grouped_mm_bf16: n or k too large for 256-row tiles");
  hipLaunchKernelGGL((grouped_mm_big_kernel<F16, GLU, OutT>), dim3(G), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), m_indptr,
                     static_cast<OutT*>(out), static_cast<int>(m_rows), static_cast<int>(k),
                     static_cast<int>(n), static_cast<int>(batch), gl);
  return launch_status(GLU ? "grouped_mm_swiglu" : "grouped_mm_bf16");
}

template <bool F16, typename OutT>
mi_status dispatch_grouped(const void* a, int64_t m_rows, int64_t k, const void* b,
                           int64_t batch, int64_t n, const int32_t* m_indptr, void* out,
                           hipStream_t stream) {
  // Tile shape from host-known sizes only (the counts live on the device):
  // large average groups take 256x256 tiles; smaller groups stream b from HBM
  // and take 64x64 tiles, two workgroups per CU, with 4 K steps in flight.
  const int64_t avg = m_rows / batch;
  if (avg >= 192)
    return launch_grouped_big<F16, false, OutT>(a, m_rows, k, b, batch, n, m_indptr, out, stream,
                                               GbGlu{});
  return launch_grouped<64, 64, 64, 2, 2, 4, F16, OutT>(a, m_rows, k, b, batch, n, m_indptr, out, stream, 2);
}

}  // namespace
}  // namespace mi

extern "C" mi_status mi_grouped_mm_bf16(const void* a, int64_t m_rows, int64_t k, mi_dtype ab_dtype,
                                        const void* b, int64_t batch, int64_t n,
                                        const int32_t* m_indptr, void* out, mi_dtype out_dtype,
                                        void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(batch >= 1, "grouped_mm_bf16: batch_size must be >= 1 (got %lld)", (long long)batch);
  MI_REQUIRE(batch <= GM_MAX_EXPERTS, "grouped_mm_bf16: batch_size must be <= %d (got %lld)",
             GM_MAX_EXPERTS, (long long)batch);
  MI_REQUIRE(m_rows >= 0 && m_rows < (1LL << 31), "grouped_mm_bf16: cum_m out of range (%lld)",
             (long long)m_rows);
  MI_REQUIRE(n > 0 && n % 256 == 0, "grouped_mm_bf16: n %% 256 == 0 required (got n=%lld)",
             (long long)n);
  MI_REQUIRE(k > 0 && k % 64 == 0, "grouped_mm_bf16: k %% 64 == 0 required (got k=%lld)",
             (long long)k);
  MI_REQUIRE(n < (1LL << 31) && k < (1LL << 31), "grouped_mm_bf16: n or k too large");
  MI_REQUIRE(ab_dtype == MI_BF16 || ab_dtype == MI_F16,
             "grouped_mm_bf16: a and b must be bf16 or fp16");
  MI_REQUIRE(out_dtype == MI_BF16 || out_dtype == MI_F32 || out_dtype == MI_F16,
             "grouped_mm_bf16: out_dtype must be bf16, fp16 or fp32");
  MI_REQUIRE(m_indptr != nullptr, "grouped_mm_bf16: m_indptr is null");
  MI_REQUIRE(b != nullptr, "grouped_mm_bf16: b is null");
  if (m_rows == 0) return MI_OK;
  MI_REQUIRE(a != nullptr && out != nullptr, "grouped_mm_bf16: a/out is null");
  MI_REQUIRE(aligned16(a) && aligned16(b), "grouped_mm_bf16: a and b must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = ab_dtype == MI_F16;
  if (out_dtype == MI_BF16)
    return f16 ? dispatch_grouped<true, Bf16Out>(a, m_rows, k, b, batch, n, m_indptr, out, s)
               : dispatch_grouped<false, Bf16Out>(a, m_rows, k, b, batch, n, m_indptr, out, s);
  if (out_dtype == MI_F16)
    return f16 ? dispatch_grouped<true, _Float16>(a, m_rows, k, b, batch, n, m_indptr, out, s)
               : dispatch_grouped<false, _Float16>(a, m_rows, k, b, batch, n, m_indptr, out, s);
  return f16 ? dispatch_grouped<true, float>(a, m_rows, k, b, batch, n, m_indptr, out, s)
             : dispatch_grouped<false, float>(a, m_rows, k, b, batch, n, m_indptr, out, s);
}

extern "C" mi_status mi_grouped_mm_swiglu(const void* a, int64_t m_rows, int64_t k,
                                          mi_dtype ab_dtype, const void* b, int64_t batch,
                                          int64_t inter_size, const int32_t* m_indptr,
                                          const void* fc1_delta, const float* alpha,
                                          const float* beta, const float* limit, void* out,
                                          mi_dtype out_dtype, void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(batch >= 1 && batch <= GM_MAX_EXPERTS,
             "grouped_mm_swiglu: batch_size must be in [1, %d] (got %lld)", GM_MAX_EXPERTS,
             (long long)batch);
  MI_REQUIRE(m_rows >= 0 && m_rows < (1LL << 31), "grouped_mm_swiglu: cum_m out of range");
  MI_REQUIRE(inter_size > 0 && inter_size % 128 == 0 && inter_size < (1LL << 30),
             "grouped_mm_swiglu: intermediate size %% 128 == 0 required (got %lld)",
             (long long)inter_size);
  MI_REQUIRE(k > 0 && k % 64 == 0 && k < (1LL << 31),
             "grouped_mm_swiglu: k %% 64 == 0 required (got k=%lld)", (long long)k);
  MI_REQUIRE(ab_dtype == MI_BF16 || ab_dtype == MI_F16,
             "grouped_mm_swiglu: a and b must be bf16 or fp16");
  MI_REQUIRE(out_dtype == MI_BF16 || out_dtype == MI_F32 || out_dtype == MI_F16,
             "grouped_mm_swiglu: out_dtype must be bf16, fp16 or fp32");
  MI_REQUIRE(m_indptr != nullptr && b != nullptr, "grouped_mm_swiglu: m_indptr or b is null");
  if (m_rows == 0) return MI_OK;
  MI_REQUIRE(a != nullptr && out != nullptr, "grouped_mm_swiglu: a/out is null");
  MI_REQUIRE(aligned16(a) && aligned16(b), "grouped_mm_swiglu: a and b must be 16-byte aligned");
  MI_REQUIRE(fc1_delta == nullptr || (reinterpret_cast<uintptr_t>(fc1_delta) & 7) == 0,
             "grouped_mm_swiglu: fc1_delta must be 8-byte aligned");
  MI_REQUIRE((reinterpret_cast<uintptr_t>(out) & 15) == 0,
             "grouped_mm_swiglu: out must be 16-byte aligned");
  const int64_t n = 2 * inter_size;
  const GbGlu gl{static_cast<const uint16_t*>(fc1_delta), alpha, beta, limit};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = ab_dtype == MI_F16;
  if (out_dtype == MI_BF16)
    return f16 ? launch_grouped_big<true, true, Bf16Out>(a, m_rows, k, b, batch, n, m_indptr, out, s, gl)
               : launch_grouped_big<false, true, Bf16Out>(a, m_rows, k, b, batch, n, m_indptr, out, s, gl);
  if (out_dtype == MI_F16)
    return f16 ? launch_grouped_big<true, true, _Float16>(a, m_rows, k, b, batch, n, m_indptr, out, s, gl)
               : launch_grouped_big<false, true, _Float16>(a, m_rows, k, b, batch, n, m_indptr, out, s, gl);
  return f16 ? launch_grouped_big<true, true, float>(a, m_rows, k, b, batch, n, m_indptr, out, s, gl)
             : launch_grouped_big<false, true, float>(a, m_rows, k, b, batch, n, m_indptr, out, s, gl);
}
