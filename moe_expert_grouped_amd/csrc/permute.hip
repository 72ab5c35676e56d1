// Routing output -> expert-sorted permutation, and the permuted rows, on gfx950.
//
// expanded_idx_to_permuted_idx maps the expanded index token*top_k + slot to
// the permuted row, negative for an inactive slot (flashinfer.fused_moe.
// bgmv_moe_gemm2_lora_delta, parameters); m_indptr holds the cumulative row
// counts of the groups, one per expert (flashinfer.grouped_mm.grouped_mm_bf16,
// parameters).  The permuted order is a stable sort of the expanded slots by
// expert id; a slot whose id lies outside [0, num_experts) is not routed here.
//
// mi_moe_route_permutation is a stable counting sort of the N = T*top_k slots
// in three launches and no host reads.  The slots are cut in chunks of
// RP_CHUNK; the workspace holds cnt[e][c], expert-major.
//  1. count  (one workgroup per chunk) -- cnt[e][c] = slots of chunk c routed
//            to e (LDS atomics: the order does not matter here).
//  2. scan   (one workgroup) -- an exclusive scan of cnt over its flat,
//            expert-major order turns cnt[e][c] into the first row of chunk
//            c's slots of expert e: all rows of experts below e, then those of
//            e's earlier chunks.  Its values at c = 0 are m_indptr.
//  3. place  (one wavefront per chunk) -- walks the chunk's slots 64 at a
//            time, in order.  Lanes holding the same expert find each other
//            with one ballot per id bit; a lane's row is the running row of
//            its expert plus the count of such lanes below it, and the highest
//            lane of the group advances the running row.  Stable, and the
//            result does not depend on the order the chunks run in.
// mi_moe_permute_rows copies each token row once from HBM and writes it to
// the permuted rows of the token's slots (one wavefront per token).
#include "common.hpp"

namespace mi {
namespace {

constexpr int RP_CHUNK = 1024;  // slots per chunk
constexpr int RP_PER_LANE = RP_CHUNK / 64;
constexpr int RP_MAX_EXPERTS = 1024;
constexpr int RP_ID_BITS = 11;  // ids 0 .. 1023 and the "not routed here" mark
constexpr int RP_NOT_HERE = (1 << RP_ID_BITS) - 1;
constexpr int SCAN_THREADS = 1024;
constexpr int ROWS_UNROLL = 4;  // 16-byte pieces per lane in flight

int64_t rp_chunks(int64_t n) { return (n + RP_CHUNK - 1) / RP_CHUNK; }

__global__ __launch_bounds__(256) void rp_count_kernel(const int32_t* __restrict__ ids, int n,
                                                       int E, int nch,
                                                       int32_t* __restrict__ cnt) {
  __shared__ int s_cnt[RP_MAX_EXPERTS];
  const int c = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) s_cnt[e] = 0;
  __syncthreads();
  const int x0 = c * RP_CHUNK, x1 = min(n, x0 + RP_CHUNK);
  for (int x = x0 + tid; x < x1; x += 256) {
    const int id = gld<int>(ids + x);
    if (id >= 0 && id < E) atomicAdd(&s_cnt[id], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) gst<int>(cnt + static_cast<int64_t>(e) * nch + c, s_cnt[e]);
}

// In-place exclusive scan of cnt[0 .. E*nch), 4 consecutive values per thread
// per pass; writes m_indptr and marks inverse[total .. n) with -1.
__global__ __launch_bounds__(SCAN_THREADS) void rp_scan_kernel(int32_t* __restrict__ cnt,
                                                               int64_t m, int nch, int E, int n,
                                                               int32_t* __restrict__ m_indptr,
                                                               int32_t* __restrict__ inverse) {
  __shared__ int s_wsum[SCAN_THREADS / 64];
  __shared__ int s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < m; base += 4 * SCAN_THREADS) {
    const int64_t i0 = base + 4 * static_cast<int64_t>(tid);
    int v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i0 + u < m ? gld<int>(cnt + i0 + u) : 0;
    const int own = v[0] + v[1] + v[2] + v[3];
    int incl = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int run = s_carry;
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
    run += incl - own;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u;
      if (i < m) {
        gst<int>(cnt + i, run);
        if (i % nch == 0) gst<int>(m_indptr + i / nch, run);
      }
      run += v[u];
    }
    __syncthreads();  // every thread has read s_carry and s_wsum
    if (tid == SCAN_THREADS - 1) s_carry = run;
    __syncthreads();
  }
  const int total = s_carry;
  if (tid == 0) gst<int>(m_indptr + E, total);
  if (m == 0)
    for (int e = tid; e < E; e += SCAN_THREADS) gst<int>(m_indptr + e, 0);
  if (inverse != nullptr)
    for (int p = total + tid; p < n; p += SCAN_THREADS) gst<int>(inverse + p, -1);
}

__global__ __launch_bounds__(64) void rp_place_kernel(const int32_t* __restrict__ ids, int n,
                                                      int E, int nch,
                                                      const int32_t* __restrict__ first,
                                                      int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ inverse) {
  __shared__ int s_row[RP_MAX_EXPERTS];
  const int c = blockIdx.x, lane = threadIdx.x;
  const int x0 = c * RP_CHUNK;
  int v[RP_PER_LANE];
#pragma unroll
  for (int i = 0; i < RP_PER_LANE; ++i) {
    const int x = x0 + 64 * i + lane;
    const int id = x < n ? gld<int>(ids + x) : -1;
    v[i] = id >= 0 && id < E ? id : RP_NOT_HERE;
  }
  for (int e = lane; e < E; e += 64) s_row[e] = gld<int>(first + static_cast<int64_t>(e) * nch + c);
  __builtin_amdgcn_wave_barrier();
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < RP_PER_LANE; ++i) {
    const int x = x0 + 64 * i + lane;
    // lanes holding the same value: for each bit, keep the lanes that agree
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < RP_ID_BITS; ++b) {
      const bool bit = (v[i] >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const bool routed = v[i] != RP_NOT_HERE;
    int pos = -1;
    if (routed) pos = s_row[v[i]] + __popcll(peers & below);
    if (x < n) {
      gst<int>(perm + x, pos);
      // pos < n holds when the ids did not change between the launches
      if (routed && inverse != nullptr && pos < n) gst<int>(inverse + pos, x);
    }
    // LDS operations of one wavefront complete in order: every read above
    // sees the running rows before this update
    __builtin_amdgcn_wave_barrier();
    if (routed && (peers >> lane) == 1ull) s_row[v[i]] = pos + 1;
    __builtin_amdgcn_wave_barrier();
  }
}

// One wavefront per token: the row is read once, in pieces of 64*ROWS_UNROLL
// 16-byte chunks, and stored to each of the token's permuted rows.
__global__ __launch_bounds__(256) void rp_rows_kernel(const uint8_t* __restrict__ x, int T,
                                                      int64_t cpr, const int32_t* __restrict__ perm,
                                                      int top_k, int64_t out_rows,
                                                      uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    const uint8_t* src = x + static_cast<int64_t>(t) * cpr * 16;
    for (int64_t c0 = 0; c0 < cpr; c0 += 64 * ROWS_UNROLL) {
      u32x4 d[ROWS_UNROLL];
#pragma unroll
      for (int u = 0; u < ROWS_UNROLL; ++u) {
        const int64_t c = c0 + 64 * u + lane;
        if (c < cpr) d[u] = gld<u32x4>(src + c * 16);
      }
      for (int j = 0; j < top_k; ++j) {
        const int p = gld<int>(perm + static_cast<int64_t>(t) * top_k + j);
        if (p < 0 || p >= out_rows) continue;
        uint8_t* dst = out + static_cast<int64_t>(p) * cpr * 16;
#pragma unroll
        for (int u = 0; u < ROWS_UNROLL; ++u) {
          const int64_t c = c0 + 64 * u + lane;
          // streaming stores: the permuted rows are not read again by this kernel
          if (c < cpr) __builtin_nontemporal_store(d[u], reinterpret_cast<u32x4*>(dst + c * 16));
        }
      }
    }
  }
}

}  // namespace
}  // namespace mi

extern "C" size_t mi_moe_route_workspace_size(int64_t num_slots, int64_t num_experts) {
  if (num_slots < 0 || num_experts < 1) return 0;
  return static_cast<size_t>(mi::rp_chunks(num_slots)) * static_cast<size_t>(num_experts) * 4 + 256;
}

extern "C" mi_status mi_moe_route_permutation(const int32_t* topk_ids, int64_t num_tokens,
                                              int64_t top_k, int64_t num_experts,
                                              int32_t* m_indptr, int32_t* perm,
                                              int32_t* inverse, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(num_tokens >= 0 && top_k >= 1 && num_tokens <= (1LL << 31) / top_k - 1,
             "moe_route_permutation: num_tokens * top_k must be in [0, 2^31)");
  MI_REQUIRE(num_experts >= 1 && num_experts <= RP_MAX_EXPERTS,
             "moe_route_permutation: num_experts must be in [1, %d] (got %lld)", RP_MAX_EXPERTS,
             (long long)num_experts);
  MI_REQUIRE(m_indptr != nullptr, "moe_route_permutation: m_indptr is null");
  const int64_t n = num_tokens * top_k;
  const int64_t nch = rp_chunks(n);
  MI_REQUIRE(n == 0 || (topk_ids != nullptr && perm != nullptr),
             "moe_route_permutation: topk_ids or expanded_idx_to_permuted_idx is null");
  const size_t need = mi_moe_route_workspace_size(n, num_experts);
  MI_REQUIRE(workspace != nullptr && workspace_bytes >= need,
             "moe_route_permutation: the workspace needs %zu bytes (got %zu)", need,
             workspace_bytes);
  MI_REQUIRE(nch <= 0x7fffffff / 64, "moe_route_permutation: too many slots");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* cnt = static_cast<int32_t*>(workspace);
  const int E = static_cast<int>(num_experts), ni = static_cast<int>(n);
  const int nc = static_cast<int>(nch);
  if (nch > 0) {
    hipLaunchKernelGGL(rp_count_kernel, dim3(static_cast<unsigned>(nch)), dim3(256), 0, s,
                       topk_ids, ni, E, nc, cnt);
    const mi_status st = launch_status("moe_route_permutation (count)");
    if (st != MI_OK) return st;
  }
  hipLaunchKernelGGL(rp_scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, cnt, nch * E,
                     nc > 0 ? nc : 1, E, ni, m_indptr, inverse);
  const mi_status st = launch_status("moe_route_permutation (scan)");
  if (st != MI_OK || nch == 0) return st;
  hipLaunchKernelGGL(rp_place_kernel, dim3(static_cast<unsigned>(nch)), dim3(64), 0, s, topk_ids,
                     ni, E, nc, cnt, perm, inverse);
  return launch_status("moe_route_permutation (place)");
}

extern "C" mi_status mi_moe_permute_rows(const void* x, int64_t num_tokens, int64_t row_bytes,
                                         const int32_t* perm, int64_t top_k, void* out,
                                         int64_t out_rows, void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(num_tokens >= 0 && num_tokens < (1LL << 31) && top_k >= 1 &&
                 num_tokens <= (1LL << 31) / top_k - 1,
             "moe_permute_rows: num_tokens * top_k must be in [0, 2^31)");
  MI_REQUIRE(row_bytes > 0 && row_bytes % 16 == 0,
             "moe_permute_rows: row_bytes must be a positive multiple of 16 (got %lld)",
             (long long)row_bytes);
  MI_REQUIRE(out_rows >= 0, "moe_permute_rows: out_rows must be >= 0");
  if (num_tokens == 0 || out_rows == 0) return MI_OK;
  MI_REQUIRE(x != nullptr && perm != nullptr && out != nullptr, "moe_permute_rows: null pointer");
  MI_REQUIRE(aligned16(x) && aligned16(out),
             "moe_permute_rows: x and out must be 16-byte aligned");
  int64_t blocks = (num_tokens + 3) / 4;
  if (blocks > 8192) blocks = 8192;  // the wavefronts stride over the tokens beyond
  hipLaunchKernelGGL(rp_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(x),
                     static_cast<int>(num_tokens), row_bytes / 16, perm, static_cast<int>(top_k),
                     out_rows, static_cast<uint8_t*>(out));
  return launch_status("moe_permute_rows");
}
