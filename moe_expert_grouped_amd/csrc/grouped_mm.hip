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
// Kernel structure
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

template <bool F16, typename OutT>
mi_status dispatch_grouped(const void* a, int64_t m_rows, int64_t k, const void* b,
                           int64_t batch, int64_t n, const int32_t* m_indptr, void* out,
                           hipStream_t stream) {
  // Tile shape from host-known sizes only (the counts live on the device):
  // large average groups take 256x256 tiles; smaller groups stream b from HBM
  // and take 64x64 tiles, two workgroups per CU, with 4 K steps in flight.
  const int64_t avg = m_rows / batch;
  if (avg >= 192)
    return launch_grouped<256, 256, 64, 4, 2, 1, F16, OutT>(a, m_rows, k, b, batch, n, m_indptr, out, stream,
                                                   1);
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
