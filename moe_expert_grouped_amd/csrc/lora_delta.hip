// FC2 LoRA delta of a routed MoE on gfx950.
//
// delta[t] = scale * sum_j w[t,j] * B_down[l,e] @ (A_down[l,e] @ act[perm[t*top_k+j]])
// (flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta, formula and parameters).
//
// Three launches on the caller's stream, no host reads:
//
//  1. plan    (one workgroup) -- decodes every slot (t, j): it is active iff
//             the permuted row p >= 0 (and < padded_rows), the adapter
//             l = lora_ids[t] lies in [0, num_adapters) and the expert lies in
//             [0, num_experts).  Active slots are bucketed by key (l, e) and
//             tokens by adapter (bucket num_adapters = "no adapter").  It emits
//             two work lists: shrink items (<= 16 slots of one key) and expand
//             items (<= TT tokens of one adapter bucket).  Positions inside a
//             bucket come from LDS atomics, so the order varies between runs;
//             no result depends on it (every slot and every token is computed
//             by the same instruction sequence wherever it lands).
//  2. shrink  -- one wavefront per shrink item: u[slot, :] = (scale*w) *
//             A_le @ act[p] with v_mfma_f32_16x16x32_bf16 (16 slots x 16 ranks,
//             K = inter_size); the act rows are gathered straight from HBM and
//             A_le is shared by the item's 16 slots.  u stays fp32.
//  3. expand  -- one workgroup per (expand item, H range): the tile's tokens
//             (one adapter, up to 32 per wavefront) walk the experts in
//             increasing order; B_le[h-chunk, :] is staged through LDS once per
//             workgroup and expert; each token contributes its slot's u for
//             that expert (zero when it has none) as the MFMA A operand.  u is
//             split exactly-enough into bf16 hi + lo parts (two MFMAs), so the
//             intermediate keeps ~16 significand bits.  Accumulation per token
//             runs over experts in a fixed order: bitwise repeatable.  Tokens
//             of the "no adapter" bucket get +0 rows.
#include "common.hpp"

namespace mi {
namespace {

constexpr int PLAN_THREADS = 1024;
constexpr int MAX_KEYS = 8192;      // num_adapters * num_experts
constexpr int MAX_ADAPTERS = 1023;  // + 1 "none" bucket
constexpr int SHRINK_ROWS = 16;
constexpr int EXP_TOK_PER_WAVE = 32;
constexpr int EXP_HC = 128;         // H columns per expand pass (4 x 32 per wave)
constexpr int MAX_TOPK = 32;

struct Item {  // a run of sorted entries
  int start, count, key, pad;
};

struct Layout {
  size_t u, slot_list, tok_list, shrink_items, expand_items, counters, total;
};

__host__ __device__ inline size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int expand_waves(int64_t top_k, int64_t rank) {
  // LDS per token: top_k * rank * 4 bytes (bf16 hi + lo); budget 64 KiB
  const int64_t per_tok = top_k * rank * 4;
  int64_t w = (64 * 1024) / (EXP_TOK_PER_WAVE * per_tok);
  if (w > 4) w = 4;
  return static_cast<int>(w);
}

Layout layout(int64_t T, int64_t top_k, int64_t E, int64_t L, int64_t rank) {
  Layout ly{};
  const int64_t slots = T * top_k;
  const int ew = expand_waves(top_k, rank);
  const int64_t tt = (ew > 0 ? ew : 1) * EXP_TOK_PER_WAVE;
  size_t off = 0;
  ly.u = off;
  off = al256(off + static_cast<size_t>(slots * rank) * 4);
  ly.slot_list = off;
  off = al256(off + static_cast<size_t>(slots) * 4);
  ly.tok_list = off;
  off = al256(off + static_cast<size_t>(T) * 4);
  ly.shrink_items = off;
  off = al256(off + static_cast<size_t>(slots / SHRINK_ROWS + L * E + 1) * sizeof(Item));
  ly.expand_items = off;
  off = al256(off + static_cast<size_t>(T / tt + L + 2) * sizeof(Item));
  ly.counters = off;
  off = al256(off + 64);
  ly.total = off;
  return ly;
}

// ---------------------------------------------------------------------------
// 1. plan
// ---------------------------------------------------------------------------
struct PlanArgs {
  const int32_t* perm;
  const int32_t* topk_ids;
  const int32_t* lora_ids;
  int T, top_k, E, L, padded_rows, tok_tile;
  int32_t* slot_list;
  int32_t* tok_list;
  Item* shrink_items;
  Item* expand_items;
  int32_t* counters;  // [0] shrink item count, [1] expand item count
};

__device__ __forceinline__ int slot_key(const PlanArgs& p, int x) {
  const int t = x / p.top_k;
  const int l = p.lora_ids[t];
  const int r = p.perm[x];
  const int e = p.topk_ids[x];
  if (l < 0 || l >= p.L || r < 0 || r >= p.padded_rows || e < 0 || e >= p.E) return -1;
  return l * p.E + e;
}

// exclusive scan of n ints in LDS (in place), returns the total; all threads call
__device__ int block_exclusive_scan(int* v, int n, int* s_part) {
  const int tid = threadIdx.x;
  const int per = (n + PLAN_THREADS - 1) / PLAN_THREADS;
  const int b0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < n) local += v[b0 + i];
  // wave inclusive scan
  const int lane = tid & 63, wave = tid >> 6;
  int incl = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_part[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < PLAN_THREADS / 64; ++w) {
      const int c = s_part[w];
      s_part[w] = run;
      run += c;
    }
    s_part[PLAN_THREADS / 64] = run;
  }
  __syncthreads();
  int run = s_part[wave] + incl - local;
  for (int i = 0; i < per; ++i)
    if (b0 + i < n) {
      const int c = v[b0 + i];
      v[b0 + i] = run;
      run += c;
    }
  const int total = s_part[PLAN_THREADS / 64];
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(PlanArgs p) {
  __shared__ int s_cnt[MAX_KEYS];
  __shared__ int s_off[MAX_KEYS];
  __shared__ int s_blk[MAX_KEYS];
  __shared__ int s_tcnt[MAX_ADAPTERS + 1];
  __shared__ int s_toff[MAX_ADAPTERS + 1];
  __shared__ int s_tblk[MAX_ADAPTERS + 1];
  __shared__ int s_part[PLAN_THREADS / 64 + 1];
  const int tid = threadIdx.x;
  const int nkeys = p.L * p.E;
  const int nb = p.L + 1;
  const int slots = p.T * p.top_k;

  for (int i = tid; i < nkeys; i += PLAN_THREADS) s_cnt[i] = 0;
  for (int i = tid; i < nb; i += PLAN_THREADS) s_tcnt[i] = 0;
  __syncthreads();
  for (int x = tid; x < slots; x += PLAN_THREADS) {
    const int key = slot_key(p, x);
    if (key >= 0) atomicAdd(&s_cnt[key], 1);
  }
  for (int t = tid; t < p.T; t += PLAN_THREADS) {
    const int l = p.lora_ids[t];
    atomicAdd(&s_tcnt[(l >= 0 && l < p.L) ? l : p.L], 1);
  }
  __syncthreads();
  for (int i = tid; i < nkeys; i += PLAN_THREADS) {
    s_off[i] = s_cnt[i];
    s_blk[i] = (s_cnt[i] + SHRINK_ROWS - 1) / SHRINK_ROWS;
  }
  for (int i = tid; i < nb; i += PLAN_THREADS) {
    s_toff[i] = s_tcnt[i];
    s_tblk[i] = (s_tcnt[i] + p.tok_tile - 1) / p.tok_tile;
  }
  __syncthreads();
  block_exclusive_scan(s_off, nkeys, s_part);
  const int n_shrink = block_exclusive_scan(s_blk, nkeys, s_part);
  block_exclusive_scan(s_toff, nb, s_part);
  const int n_expand = block_exclusive_scan(s_tblk, nb, s_part);

  for (int key = tid; key < nkeys; key += PLAN_THREADS) {
    const int c = s_cnt[key];
    for (int b = 0; b * SHRINK_ROWS < c; ++b)
      p.shrink_items[s_blk[key] + b] = Item{s_off[key] + b * SHRINK_ROWS,
                                            min(SHRINK_ROWS, c - b * SHRINK_ROWS), key, 0};
  }
  for (int bk = tid; bk < nb; bk += PLAN_THREADS) {
    const int c = s_tcnt[bk];
    for (int b = 0; b * p.tok_tile < c; ++b)
      p.expand_items[s_tblk[bk] + b] =
          Item{s_toff[bk] + b * p.tok_tile, min(p.tok_tile, c - b * p.tok_tile), bk, 0};
  }
  if (tid == 0) {
    p.counters[0] = n_shrink;
    p.counters[1] = n_expand;
  }
  __syncthreads();
  // scatter (cursor = running offsets)
  for (int x = tid; x < slots; x += PLAN_THREADS) {
    const int key = slot_key(p, x);
    if (key >= 0) p.slot_list[atomicAdd(&s_off[key], 1)] = x;
  }
  for (int t = tid; t < p.T; t += PLAN_THREADS) {
    const int l = p.lora_ids[t];
    p.tok_list[atomicAdd(&s_toff[(l >= 0 && l < p.L) ? l : p.L], 1)] = t;
  }
}

// ---------------------------------------------------------------------------
// 2. shrink
// ---------------------------------------------------------------------------
struct ShrinkArgs {
  const uint16_t* act;
  const int32_t* perm;
  const int64_t* w_ptr_a;
  long stride_a;
  const float* topk_weights;
  const int32_t* slot_list;
  const Item* items;
  const int32_t* counters;
  float* u;
  int I, E, rank;
  float scale;
};

template <int NB>  // number of 16-rank blocks
__global__ __launch_bounds__(256) void shrink_kernel(ShrinkArgs p) {
  const int lane = threadIdx.x & 63;
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  const int n_items = p.counters[0];
  const int row = lane & 15, kq = lane >> 4;  // k offset 8*kq inside a 32-wide step
  for (int it = gw; it < n_items; it += nw) {
    const Item item = p.items[it];
    const int l = item.key / p.E, e = item.key % p.E;
    const int x = p.slot_list[item.start + min(row, item.count - 1)];
    const uint16_t* arow = p.act + static_cast<long>(p.perm[x]) * p.I + kq * 8;
    const uint16_t* Ale = reinterpret_cast<const uint16_t*>(p.w_ptr_a[e]) +
                          static_cast<long>(l) * p.stride_a;
    const uint16_t* brow[NB];
    bool bvalid[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int rr = nb * 16 + row;
      bvalid[nb] = rr < p.rank;
      brow[nb] = Ale + static_cast<long>(bvalid[nb] ? rr : 0) * p.I + kq * 8;
    }
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int I = p.I;
    int k0 = 0;
    constexpr int U = 4;
    for (; k0 + 32 * U <= I; k0 += 32 * U) {
      u32x4 fa[U], fb[U][NB];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        fa[uu] = *reinterpret_cast<const u32x4*>(arow + k0 + 32 * uu);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          fb[uu][nb] = bvalid[nb] ? *reinterpret_cast<const u32x4*>(brow[nb] + k0 + 32 * uu)
                                  : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[uu]),
                                                            __builtin_bit_cast(bf16x8, fb[uu][nb]),
                                                            acc[nb], 0, 0, 0);
    }
    for (; k0 < I; k0 += 32) {
      const bool kin = k0 + kq * 8 < I;  // I % 8 == 0
      const u32x4 fa = kin ? *reinterpret_cast<const u32x4*>(arow + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 fb = (kin && bvalid[nb]) ? *reinterpret_cast<const u32x4*>(brow[nb] + k0)
                                             : u32x4{0, 0, 0, 0};
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, fa), __builtin_bit_cast(bf16x8, fb), acc[nb], 0, 0, 0);
      }
    }
    // acc[nb][q] = u_raw[slot row 4*kq + q][rank nb*16 + row]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int srow = 4 * kq + q;
      if (srow < item.count) {
        const int xs = p.slot_list[item.start + srow];
        const float f = p.scale * p.topk_weights[xs];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int rr = nb * 16 + row;
          if (rr < p.rank) p.u[static_cast<long>(xs) * p.rank + rr] = acc[nb][q] * f;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. expand
// ---------------------------------------------------------------------------
struct ExpandArgs {
  const int32_t* perm;
  const int32_t* topk_ids;
  const int64_t* w_ptr_b;
  long stride_b;
  const int32_t* tok_list;
  const Item* items;
  const int32_t* counters;
  const float* u;
  void* out;
  int T, top_k, E, L, H, rank, padded_rows;
  int out_f32;
  int h_splits;  // H ranges per item
};

__device__ __forceinline__ void split_hi_lo(float v, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(v);
  lo = f32_to_bf16_rne(v - bf16_bits_to_f32(hi));
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void expand_kernel(ExpandArgs p) {
  constexpr int TT = NW * EXP_TOK_PER_WAVE;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsmem[];
  // [TT][top_k] sorted expert ids (int32), [TT][top_k][2][rank] bf16 hi/lo u,
  // 2 x [EXP_HC][rank] bf16 B stage
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.top_k, R = p.rank;
  int32_t* s_eid = reinterpret_cast<int32_t*>(dsmem);
  uint16_t* s_u = reinterpret_cast<uint16_t*>(dsmem + al256(TT * K * 4));
  uint16_t* s_b = s_u + static_cast<long>(TT) * K * 2 * R;
  __shared__ int s_ntok;

  const int n_items = p.counters[1];
  const long total = static_cast<long>(n_items) * p.h_splits;
  const int hrange = p.H / p.h_splits;  // multiple of EXP_HC or the whole H
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    const Item item = p.items[w / p.h_splits];
    const int hs = static_cast<int>(w % p.h_splits);
    const int h_begin = hs * hrange, h_end = h_begin + hrange;
    __syncthreads();  // LDS reuse across iterations

    if (item.key >= p.L) {  // no adapter: +0 rows
      for (int i = wave; i < item.count; i += NW) {
        const int t = p.tok_list[item.start + i];
        for (int h = h_begin + lane * 4; h < h_end; h += 256) {
          if (p.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + static_cast<long>(t) * p.H + h) =
                f32x4{0.f, 0.f, 0.f, 0.f};
          } else {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + static_cast<long>(t) * p.H +
                                      h) = make_uint2(0u, 0u);
          }
        }
      }
      continue;
    }
    const int l = item.key;

    // ---- setup: per token, its active slots sorted by expert, u as bf16 hi/lo ----
    for (int i = tid; i < TT; i += 64 * NW) {
      int32_t* te = s_eid + i * K;
      uint16_t* tu = s_u + static_cast<long>(i) * K * 2 * R;
      int n = 0;
      if (i < item.count) {
        const int t = p.tok_list[item.start + i];
        for (int j = 0; j < K; ++j) {  // insertion sort of (expert, slot) keys
          const int x = t * K + j;
          const int e = p.topk_ids[x], r = p.perm[x];
          if (r < 0 || r >= p.padded_rows || e < 0 || e >= p.E) continue;
          const int key = (e << 5) | j;
          int pos = n++;
          while (pos > 0 && te[pos - 1] > key) {
            te[pos] = te[pos - 1];
            --pos;
          }
          te[pos] = key;
        }
        // merge slots of the same expert (their u are summed), store hi/lo
        int m = 0;
        for (int a = 0; a < n; ++a) {
          const int key = te[a];
          const int e = key >> 5, j = key & 31;
          const float* us = p.u + static_cast<long>(t * K + j) * R;
          if (m > 0 && te[m - 1] == e) {
            uint16_t* dst = tu + (m - 1) * 2 * R;
            for (int rr = 0; rr < R; ++rr) {
              const float prev = bf16_bits_to_f32(dst[rr]) + bf16_bits_to_f32(dst[R + rr]);
              uint32_t hi, lo;
              split_hi_lo(prev + us[rr], hi, lo);
              dst[rr] = static_cast<uint16_t>(hi);
              dst[R + rr] = static_cast<uint16_t>(lo);
            }
            continue;
          }
          te[m] = e;  // m <= a: entry a was read above
          uint16_t* dst = tu + m * 2 * R;
          for (int rr = 0; rr < R; ++rr) {
            uint32_t hi, lo;
            split_hi_lo(us[rr], hi, lo);
            dst[rr] = static_cast<uint16_t>(hi);
            dst[R + rr] = static_cast<uint16_t>(lo);
          }
          ++m;
        }
        n = m;
      }
      for (int a = n; a < K; ++a) te[a] = 0x7fffffff;  // sentinel
    }
    __syncthreads();

    // ---- per wave: 32 tokens; lane -> token lane%32, rank half kl ----
    const int tl = wave * EXP_TOK_PER_WAVE + (lane & 31);
    const int kl = lane >> 5;
    const int32_t* my_e = s_eid + tl * K;
    const uint16_t* my_u = s_u + static_cast<long>(tl) * K * 2 * R;

    for (int h0 = h_begin; h0 < h_end; h0 += EXP_HC) {
      f32x16 acc[EXP_HC / 32];
#pragma unroll
      for (int hb = 0; hb < EXP_HC / 32; ++hb)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[hb][q] = 0.f;
      int ptr = 0;
      int next_e = my_e[0];

      const long bchunk = static_cast<long>(EXP_HC) * R;  // elements per expert chunk
      // stage expert 0
      auto stage = [&](int e, int buf) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(p.w_ptr_b[e]) +
                              static_cast<long>(l) * p.stride_b + static_cast<long>(h0) * R;
        uint16_t* dst = s_b + buf * bchunk;
        for (long c = tid * 8; c < bchunk; c += 64 * NW * 8)
          *reinterpret_cast<u32x4*>(dst + c) = *reinterpret_cast<const u32x4*>(src + c);
      };
      __syncthreads();
      stage(0, 0);
      __syncthreads();
      for (int e = 0; e < p.E; ++e) {
        const int buf = e & 1;
        if (e + 1 < p.E) stage(e + 1, buf ^ 1);
        const bool has = (next_e == e);
        const uint16_t* ub = my_u + ptr * 2 * R;
        const uint16_t* sb = s_b + buf * bchunk;
        for (int r0 = 0; r0 < R; r0 += 16) {
          u32x4 hi = {0, 0, 0, 0}, lo = {0, 0, 0, 0};
          const bool kin = r0 + kl * 8 < R;
          if (has && kin) {
            hi = *reinterpret_cast<const u32x4*>(ub + r0 + kl * 8);
            lo = *reinterpret_cast<const u32x4*>(ub + R + r0 + kl * 8);
          }
#pragma unroll
          for (int hb = 0; hb < EXP_HC / 32; ++hb) {
            u32x4 fb = {0, 0, 0, 0};
            if (kin)
              fb = *reinterpret_cast<const u32x4*>(sb + static_cast<long>(hb * 32 + (lane & 31)) * R +
                                                   r0 + kl * 8);
            acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hi),
                                                              __builtin_bit_cast(bf16x8, fb),
                                                              acc[hb], 0, 0, 0);
            acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lo),
                                                              __builtin_bit_cast(bf16x8, fb),
                                                              acc[hb], 0, 0, 0);
          }
        }
        if (has) {
          ++ptr;
          next_e = ptr < K ? my_e[ptr] : 0x7fffffff;
        }
        __syncthreads();
      }
      // ---- store: token row = 8*(q/4) + 4*(lane/32) + q%4 of the wave, col lane%32 ----
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int tr = wave * EXP_TOK_PER_WAVE + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (tr < item.count) {
          const int t = p.tok_list[item.start + tr];
#pragma unroll
          for (int hb = 0; hb < EXP_HC / 32; ++hb) {
            const long o = static_cast<long>(t) * p.H + h0 + hb * 32 + (lane & 31);
            if (p.out_f32)
              static_cast<float*>(p.out)[o] = acc[hb][q];
            else
              static_cast<uint16_t*>(p.out)[o] = static_cast<uint16_t>(f32_to_bf16_rne(acc[hb][q]));
          }
        }
      }
    }
  }
}

int num_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  return v;
}

}  // namespace
}  // namespace mi

extern "C" size_t mi_moe_fc2_lora_delta_workspace_size(int64_t num_tokens, int64_t top_k,
                                                       int64_t num_experts, int64_t num_adapters,
                                                       int64_t rank) {
  if (num_tokens < 0 || top_k < 1 || num_experts < 1 || num_adapters < 0 || rank < 1) return 0;
  return mi::layout(num_tokens, top_k, num_experts, num_adapters, rank).total;
}

extern "C" mi_status mi_moe_fc2_lora_delta(
    const void* act, int64_t padded_rows, int64_t inter_size, const int32_t* perm,
    const int64_t* w_ptr_a, int64_t lora_stride_a, const int64_t* w_ptr_b, int64_t lora_stride_b,
    const int32_t* topk_ids, const float* topk_weights, const int32_t* lora_ids, int64_t T,
    int64_t top_k, int64_t E, int64_t L, int64_t rank, int64_t H, mi_dtype lora_dtype, float scale,
    mi_dtype out_dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(T >= 0 && T < (1LL << 26), "bgmv_moe_gemm2_lora_delta: num_tokens out of range");
  MI_REQUIRE(top_k >= 1 && top_k <= MAX_TOPK, "bgmv_moe_gemm2_lora_delta: top_k must be in [1, %d]",
             MAX_TOPK);
  MI_REQUIRE(E >= 1 && E <= 32767, "bgmv_moe_gemm2_lora_delta: num_experts must be in [1, 32767]");
  MI_REQUIRE(L >= 0 && L <= MAX_ADAPTERS,
             "bgmv_moe_gemm2_lora_delta: num_adapters must be in [0, %d]", MAX_ADAPTERS);
  MI_REQUIRE(L * E <= MAX_KEYS,
             "bgmv_moe_gemm2_lora_delta: num_adapters * num_experts must be <= %d", MAX_KEYS);
  MI_REQUIRE(rank >= 8 && rank <= 128 && rank % 8 == 0,
             "bgmv_moe_gemm2_lora_delta: rank must be a multiple of 8 in [8, 128] (got %lld)",
             (long long)rank);
  MI_REQUIRE(inter_size >= 8 && inter_size % 8 == 0 && inter_size < (1 << 30),
             "bgmv_moe_gemm2_lora_delta: I = gemm1_activation_output.shape[1] must be a positive "
             "multiple of 8 (got %lld)", (long long)inter_size);
  MI_REQUIRE(H >= 1 && H < (1 << 30), "bgmv_moe_gemm2_lora_delta: hidden_size out of range");
  MI_REQUIRE_SUPPORTED(H % 128 == 0,
                       "bgmv_moe_gemm2_lora_delta: hidden_size must be a multiple of 128 (got %lld)",
                       (long long)H);
  MI_REQUIRE(lora_stride_a >= 0 && lora_stride_a % 8 == 0 && lora_stride_b >= 0 &&
                 lora_stride_b % 8 == 0,
             "bgmv_moe_gemm2_lora_delta: lora strides must be non-negative multiples of 8 "
             "elements (16-byte aligned adapter blocks)");
  MI_REQUIRE(padded_rows >= 0 && padded_rows < (1LL << 31),
             "bgmv_moe_gemm2_lora_delta: padded_rows out of range");
  MI_REQUIRE_SUPPORTED(lora_dtype == MI_BF16, "bgmv_moe_gemm2_lora_delta: lora_dtype must be bf16");
  MI_REQUIRE(out_dtype == MI_BF16 || out_dtype == MI_F32 || out_dtype == MI_F16,
             "bgmv_moe_gemm2_lora_delta: out_dtype must be bf16, fp16 or fp32");
  MI_REQUIRE_SUPPORTED(out_dtype != MI_F16, "bgmv_moe_gemm2_lora_delta: fp16 output not implemented");
  const int ew = expand_waves(top_k, rank);
  MI_REQUIRE_SUPPORTED(ew >= 1, "bgmv_moe_gemm2_lora_delta: top_k * rank must be <= 512");
  if (T == 0) return MI_OK;
  MI_REQUIRE(out != nullptr, "bgmv_moe_gemm2_lora_delta: out is null");
  MI_REQUIRE(aligned16(out), "bgmv_moe_gemm2_lora_delta: out must be 16-byte aligned");
  MI_REQUIRE(lora_ids != nullptr && topk_ids != nullptr && topk_weights != nullptr &&
                 perm != nullptr,
             "bgmv_moe_gemm2_lora_delta: index/weight tensors must be non-null");
  if (L > 0)
    MI_REQUIRE(act != nullptr && w_ptr_a != nullptr && w_ptr_b != nullptr,
               "bgmv_moe_gemm2_lora_delta: act and the pointer tables must be non-null");
  MI_REQUIRE(aligned16(act), "bgmv_moe_gemm2_lora_delta: activation rows must be 16-byte aligned");
  const Layout ly = layout(T, top_k, E, L, rank);
  MI_REQUIRE(workspace != nullptr && workspace_bytes >= ly.total,
             "bgmv_moe_gemm2_lora_delta: workspace needs %zu bytes (got %zu)", ly.total,
             workspace_bytes);
  MI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255) == 0,
             "bgmv_moe_gemm2_lora_delta: workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* u = reinterpret_cast<float*>(ws + ly.u);
  int32_t* slot_list = reinterpret_cast<int32_t*>(ws + ly.slot_list);
  int32_t* tok_list = reinterpret_cast<int32_t*>(ws + ly.tok_list);
  Item* shrink_items = reinterpret_cast<Item*>(ws + ly.shrink_items);
  Item* expand_items = reinterpret_cast<Item*>(ws + ly.expand_items);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + ly.counters);
  const int tt = ew * EXP_TOK_PER_WAVE;

  PlanArgs pa{perm, topk_ids, lora_ids, static_cast<int>(T), static_cast<int>(top_k),
              static_cast<int>(E), static_cast<int>(L), static_cast<int>(padded_rows), tt,
              slot_list, tok_list, shrink_items, expand_items, counters};
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, pa);
  mi_status st = launch_status("bgmv_moe_gemm2_lora_delta (plan)");
  if (st != MI_OK) return st;

  const int cus = num_cus();
  if (L > 0) {
    ShrinkArgs sa{static_cast<const uint16_t*>(act), perm, w_ptr_a, static_cast<long>(lora_stride_a),
                  topk_weights, slot_list, shrink_items, counters, u, static_cast<int>(inter_size),
                  static_cast<int>(E), static_cast<int>(rank), scale};
    const dim3 sgrid(cus * 8), sblock(256);
    switch ((rank + 15) / 16) {
      case 1: hipLaunchKernelGGL(shrink_kernel<1>, sgrid, sblock, 0, s, sa); break;
      case 2: hipLaunchKernelGGL(shrink_kernel<2>, sgrid, sblock, 0, s, sa); break;
      case 3: hipLaunchKernelGGL(shrink_kernel<3>, sgrid, sblock, 0, s, sa); break;
      case 4: hipLaunchKernelGGL(shrink_kernel<4>, sgrid, sblock, 0, s, sa); break;
      case 5: hipLaunchKernelGGL(shrink_kernel<5>, sgrid, sblock, 0, s, sa); break;
      case 6: hipLaunchKernelGGL(shrink_kernel<6>, sgrid, sblock, 0, s, sa); break;
      case 7: hipLaunchKernelGGL(shrink_kernel<7>, sgrid, sblock, 0, s, sa); break;
      default: hipLaunchKernelGGL(shrink_kernel<8>, sgrid, sblock, 0, s, sa); break;
    }
    st = launch_status("bgmv_moe_gemm2_lora_delta (shrink)");
    if (st != MI_OK) return st;
  }

  // H split: enough workgroups to cover the chip
  int h_splits = 1;
  const int64_t est_items = T / tt + 1;
  while (H % (EXP_HC * h_splits * 2) == 0 && est_items * h_splits < 2 * cus) h_splits *= 2;
  ExpandArgs ea{perm, topk_ids, w_ptr_b, static_cast<long>(lora_stride_b), tok_list, expand_items,
                counters, u, out, static_cast<int>(T), static_cast<int>(top_k), static_cast<int>(E),
                static_cast<int>(L), static_cast<int>(H), static_cast<int>(rank),
                static_cast<int>(padded_rows), out_dtype == MI_F32 ? 1 : 0, h_splits};
  const size_t lds = al256(tt * top_k * 4) + static_cast<size_t>(tt) * top_k * 2 * rank * 2 +
                     2 * static_cast<size_t>(EXP_HC) * rank * 2;
  const dim3 egrid(cus * 2);
  static bool lds_attr_set[4] = {false, false, false, false};
  if (!lds_attr_set[ew - 1]) {
    const void* fn = ew == 1 ? reinterpret_cast<const void*>(expand_kernel<1>)
                   : ew == 2 ? reinterpret_cast<const void*>(expand_kernel<2>)
                   : ew == 3 ? reinterpret_cast<const void*>(expand_kernel<3>)
                             : reinterpret_cast<const void*>(expand_kernel<4>);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) ==
        hipSuccess)
      lds_attr_set[ew - 1] = true;
  }
  switch (ew) {
    case 1: hipLaunchKernelGGL(expand_kernel<1>, egrid, dim3(64), lds, s, ea); break;
    case 2: hipLaunchKernelGGL(expand_kernel<2>, egrid, dim3(128), lds, s, ea); break;
    case 3: hipLaunchKernelGGL(expand_kernel<3>, egrid, dim3(192), lds, s, ea); break;
    default: hipLaunchKernelGGL(expand_kernel<4>, egrid, dim3(256), lds, s, ea); break;
  }
  return launch_status("bgmv_moe_gemm2_lora_delta (expand)");
}
