// Paged decode attention on the matrix cores, for grouped-query attention
// (G query heads share one KV head; [DEEPSONAR] section 2.1) with 16-bit
// storage and head_size 128.  Same result as paged_decode_kernel (the
// definition is in that file's header); only the arithmetic layout differs.
//
// With G query heads per KV head, scoring a tile of tokens is a small dense
// product S^T[tokens x heads] = K[tokens x dims] Q^T[dims x heads], and the
// value update is O^T[dims x heads] += V^T[dims x tokens] P^T[tokens x heads].
// One 16x16 MFMA tile holds 16 tokens by 16 head columns (columns >= G carry
// a zero query and are never stored).
//
// Operand placement (lane l, column c = l % 16, group g = l / 16):
//   * Q^T (16x16x32 B operand): head c, dims 32k + 8g .. +8 — loaded once.
//   * K (16x16x32 A operand): row c of the tile is token c/4 + 4(c%4), dims
//     32k + 8g .. +8 — one 16-byte load per dim chunk k.  With that row order
//     the result S^T leaves lane l with the scores of tokens g + 4j (j < 4) of
//     head c.
//   * P^T (16x16x16 B operand): head c, tokens g + 4j — exactly the scores
//     the lane already holds, so probabilities never move between lanes.
//   * V is loaded token-major as stored (lane (g, c) reads token g + 4u,
//     dims 8c .. +8, u < 4: whole 256-byte rows), and V^T chunk e (rows =
//     dims 8m + e, k = tokens g + 4j) is two v_perm_b32 per lane away: element
//     e of each of the lane's four loads.
//   * O^T result of chunk e: head c, dims 32g + 8j + e; per head, each lane
//     group owns 32 contiguous dims.
// The online softmax is per head column: the tile max is reduced over the
// four lane groups of a column, and every accumulator of the column is
// rescaled in the lane that owns it.  P is split into a 16-bit head and a
// 16-bit remainder (P = P_hi + P_lo) so the value product keeps ~16
// significant bits of each probability.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_common.h"
#include "launch.h"
#include "pagedkv.h"

#ifndef PA_MFMA_OCCUPANCY
#define PA_MFMA_OCCUPANCY
#endif

namespace pa {
namespace {

using namespace dev;

__device__ __forceinline__ uint32_t dword(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Column c of the 16 MFMA columns is query vector c (c < NQ): new token
// c >> log2_group of the sequence (one per sequence when q_start is null) and
// query head kvh * G + (c & (G - 1)); it sees the keys below its causal bound,
// only the last W of them with a sliding window W > 0.
template <int DT, int NQ, int NW, bool FINAL>
__global__ __launch_bounds__(NW * 64) PA_MFMA_OCCUPANCY void paged_decode_mfma_kernel(
    void* __restrict__ out, const void* __restrict__ query, const void* key_cache,
    const void* value_cache, const int32_t* __restrict__ block_tables,
    int64_t bt_stride, const int32_t* __restrict__ context_lens, int32_t num_heads,
    int32_t num_kv_heads, int32_t log2_block, int32_t partition_size, int32_t num_partitions,
    float scale_log2, float* __restrict__ ws_max, float* __restrict__ ws_sum,
    float* __restrict__ ws_out, const int2* __restrict__ items, AppendArgs ap,
    const int32_t* __restrict__ shared_blocks, int32_t log2_group,
    const int32_t* __restrict__ q_start, int32_t window, int64_t num_items) {
  constexpr int D = 128;
  constexpr int DV = D / 8;   // 16-byte vectors per token row
  constexpr int NK = D / 32;  // score MFMAs per tile
  constexpr int NE = 8;       // value MFMAs per tile (dims 8m + e)
  constexpr int U = 4;        // token-major V loads per tile
  using MM = Mma<DT>;
  static_assert(NQ >= 1 && NQ <= 16, "query vectors must fit the 16 MFMA columns");

  const WorkUnit wu = work_unit(items, num_kv_heads);
  const int p = wu.p;
  const int kvh = wu.kvh;
  // A group item (sequence field < 0) serves the members of chunk -1 - s of
  // the plan's group section, which follows its items: column c holds member
  // c >> log2_group's decode query, and the partition lies in the prefix the
  // members share, read through the first member's table.  Split launches
  // only (each member's partial goes to its own workspace slot).
  const int32_t* gmem = nullptr;
  int gn = 0;
  if (wu.s < 0) {
    const int32_t* gsec = reinterpret_cast<const int32_t*>(items + num_items);
    const int c = -1 - wu.s;
    const int m0 = gsec[1 + c];
    gn = gsec[2 + c] - m0;
    gmem = gsec + 2 + gsec[0] + m0;
  }
  const int s = gmem ? gmem[0] : wu.s;
  const int L = context_lens[s];
  const int t_begin = FINAL ? 0 : p * partition_size;
  if (t_begin >= L) return;
  const int t_end = FINAL ? L : min(L, t_begin + partition_size);
  const int qlen = q_start ? q_start[s + 1] - q_start[s] : 1;
  const int nrows = gmem ? gn : qlen;  // query rows: the members, or the new tokens
  // first key any column of this sequence sees (the first new token's window)
  const int lo_min = window > 0 ? max(0, L - qlen + 1 - window) : 0;
  if (t_end <= lo_min) return;  // wholly before the window: the merge skips it

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int B = 1 << log2_block;
  const int64_t blk_stride_v = static_cast<int64_t>(num_kv_heads) * B * DV;
  const int64_t head_off_v = static_cast<int64_t>(kvh) * B * DV;
  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * bt_stride;
  // tokens of the leading blocks other sequences share (cached loads); a
  // group item reads its prefix once (streaming loads)
  const int shared_tokens = shared_blocks && !gmem ? (shared_blocks[s] << log2_block) : 0;
  if (ap.qsl && !gmem)
    apply_appends<DV, NW * 64>(ap, s, kvh, L, t_begin, t_end, bt_row, log2_block,
                                  static_cast<int64_t>(num_kv_heads) * (1 << log2_block) * DV,
                                  static_cast<int64_t>(kvh) * (1 << log2_block) * DV);
  const int h0 = kvh << log2_group;
  const int gmask = (1 << log2_group) - 1;
  const int64_t qrow0 = q_start ? q_start[s] : s;
  const int my_qi = col >> log2_group;
  const bool my_valid = col < NQ && my_qi < nrows;
  const int64_t my_row = gmem ? gmem[my_valid ? my_qi : 0] : qrow0 + my_qi;
  // keys this column sees (a member sees the whole shared prefix)
  const int bound = !my_valid ? 0 : gmem ? t_end : L - qlen + my_qi + 1;
  const int lo = window > 0 ? max(0, bound - window) : 0;   // ... from here on

  uint4 qv[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    qv[k] = make_uint4(0, 0, 0, 0);
    if (my_valid)
      qv[k] = *reinterpret_cast<const uint4*>(
          static_cast<const uint16_t*>(query) +
          (my_row * num_heads + h0 + (col & gmask)) * D + k * 32 + grp * 8);
  }

  f32x4 o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) o[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, lsum = 0.0f;

  __shared__ int32_t sm_bt[kChunkTokens];
  const uint4* kc = static_cast<const uint4*>(key_cache);
  const uint4* vc = static_cast<const uint4*>(value_cache);
  const int k_tok = (col >> 2) + 4 * (col & 3);  // token of this lane's K row

  for (int c0 = max(t_begin, lo_min); c0 < t_end; c0 += kChunkTokens) {
    const int c1 = min(c0 + kChunkTokens, t_end);
    const int b0 = c0 >> log2_block;
    const int nb = ((c1 - 1) >> log2_block) - b0 + 1;
    for (int i = threadIdx.x; i < nb; i += NW * 64) sm_bt[i] = bt_row[b0 + i];
    __syncthreads();

    const int ntiles = (c1 - c0 + kTile - 1) / kTile;
    auto vec_index = [&](int t, int vec) -> int64_t {
      const int tc = min(t, c1 - 1);
      const int32_t phys = sm_bt[(tc >> log2_block) - b0];
      const int off = tc & (B - 1);
      return static_cast<int64_t>(phys) * blk_stride_v + head_off_v + off * DV + vec;
    };

    // Tile i covers tokens c0 + 16 i ..; wave w takes tiles w, w + NW, ...
    auto load_tile = [&](auto kind, int i, uint4 (&kd)[NK], uint4 (&vd)[U]) {
      constexpr bool NT = decltype(kind)::streaming;
      const int t0 = c0 + i * kTile;
#pragma unroll
      for (int k = 0; k < NK; ++k) kd[k] = load_kv<NT>(kc + vec_index(t0 + k_tok, k * 4 + grp));
#pragma unroll
      for (int u = 0; u < U; ++u) vd[u] = load_kv<NT>(vc + vec_index(t0 + grp + 4 * u, col));
    };
    auto consume = [&](int i, const uint4 (&kr)[NK], const uint4 (&vr)[U]) {
      const int t0 = c0 + i * kTile;
      // scores of tokens grp + 4j for head col
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < NK; ++k) sc = MM::k32(kr[k], qv[k], sc);
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + grp + 4 * j;
        x[j] = (t < c1 && t < bound && t >= lo) ? sc[j] * scale_log2 : -INFINITY;
      }
      float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      const float ms = mn == -INFINITY ? 0.0f : mn;  // a column with no visible key yet
      const float corr = __builtin_amdgcn_exp2f(m - ms);
      float pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pr[j] = __builtin_amdgcn_exp2f(x[j] - ms);
      lsum = lsum * corr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      // corr is exactly 1 in a column whose maximum did not grow (and its
      // accumulators are 0 while it has seen no key): rescale only if some did
      if (__any(mn > m)) {
#pragma unroll
        for (int e = 0; e < NE; ++e) o[e] *= corr;
      }
      m = mn;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float back, unused;
        hi[j] = MM::round16(pr[j], back);
        lo[j] = MM::round16(pr[j] - back, unused);
      }
      const uint2 phi = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
      const uint2 plo = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int w = e >> 1;
        uint2 a;
        a.x = __builtin_amdgcn_perm(dword(vr[1], w), dword(vr[0], w), sel);
        a.y = __builtin_amdgcn_perm(dword(vr[3], w), dword(vr[2], w), sel);
        o[e] = MM::k16(a, phi, o[e]);
        o[e] = MM::k16(a, plo, o[e]);
      }
    };
    // A wave's tiles of one load kind, through a ring of kPrefetch + 1
    // register slots (the same pipeline as the vector kernel's).
    constexpr int NBUF = kPrefetch + 1;
    auto run = [&](auto kind, int lo_tile, int hi_tile) {
      int first, my;
      wave_tiles(lo_tile, hi_tile, wave, NW, first, my);
      uint4 kb[NBUF][NK], vb[NBUF][U];
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j)
        if (j < my) load_tile(kind, first + j * NW, kb[j], vb[j]);
      int k = 0;
      for (; k + NBUF - 1 + kPrefetch < my; k += NBUF) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          load_tile(kind, first + (k + j + kPrefetch) * NW, kb[(j + kPrefetch) % NBUF],
                    vb[(j + kPrefetch) % NBUF]);
          // keep the scheduler from sinking these loads below the consume
          __builtin_amdgcn_sched_barrier(0);
          consume(first + (k + j) * NW, kb[j], vb[j]);
        }
      }
      for (; k < my; k += NBUF) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          if (k + j < my) {
            if (k + j + kPrefetch < my)
              load_tile(kind, first + (k + j + kPrefetch) * NW, kb[(j + kPrefetch) % NBUF],
                        vb[(j + kPrefetch) % NBUF]);
            consume(first + (k + j) * NW, kb[j], vb[j]);
          }
        }
      }
    };
    // tiles that start below shared_tokens read shared blocks: cached loads
    const int n_cached = min(ntiles, max(0, (shared_tokens - c0 + kTile - 1) / kTile));
    run(LoadKind<false>{}, 0, n_cached);
    run(LoadKind<true>{}, n_cached, ntiles);
    __syncthreads();
  }

  // per-head sum of the four lane groups (disjoint token slots)
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  __shared__ float sm_m[NW][NQ];
  __shared__ float sm_l[NW][NQ];
  __shared__ float sm_acc[NW][NQ][D];
  if (col < NQ) {
    if (grp == 0) {
      sm_m[wave][col] = m;
      sm_l[wave][col] = lsum;
    }
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm_acc[wave][col][32 * grp + 8 * j + e] = o[e][j];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NQ * D; i += NW * 64) {
    const int j = i / D, d = i % D;
    const int qi = j >> log2_group;
    if (qi >= nrows) continue;  // a column past the sequence's new tokens or the members
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][j]);
    const float Ms = M == -INFINITY ? 0.0f : M;  // no visible key in this range
    float l = 0.0f, a = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = __builtin_amdgcn_exp2f(sm_m[w][j] - Ms);
      l = fmaf(sm_l[w][j], c, l);
      a = fmaf(sm_acc[w][j][d], c, a);
    }
    const int64_t row = (gmem ? gmem[qi] : qrow0 + qi) * num_heads + h0 + (j & gmask);
    if constexpr (FINAL) {
      St<DT>::store(out, row * D + d, a / l);
    } else {
      const int64_t slot = row * num_partitions + p;
      ws_out[slot * D + d] = l > 0.0f ? a / l : 0.0f;  // empty range: weight 0
      if (d == 0) {
        ws_max[slot] = M * kLn2;
        ws_sum[slot] = l;
      }
    }
  }
}

template <int DT, int NQ, bool FINAL>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = PA_MFMA_WAVES;
  int log2_block = 0;
  while ((1 << log2_block) < a.block_size) ++log2_block;
  int log2_group = 0;
  while ((1 << log2_group) < a.num_heads / a.num_kv_heads) ++log2_group;
  const dim3 grid = a.items ? dim3(static_cast<uint32_t>(a.num_items * a.num_kv_heads))
                            : dim3(FINAL ? 1 : a.num_partitions, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((paged_decode_mfma_kernel<DT, NQ, NW, FINAL>), grid, dim3(NW * 64), 0,
                     stream, a.out, a.query, a.key_cache, a.value_cache, a.block_tables,
                     a.bt_stride, a.context_lens, a.num_heads, a.num_kv_heads, log2_block,
                     a.partition_size, a.num_partitions, a.scale * kLog2e, a.ws_max, a.ws_sum,
                     a.ws_out, reinterpret_cast<const int2*>(a.items), a.append,
                     a.shared_blocks, log2_group, a.q_start, a.window, a.num_items);
  return hipGetLastError();
}

template <int DT, bool FINAL>
hipError_t dispatch_g(const DecodeArgs& a, hipStream_t stream) {
  switch (query_vectors(a)) {
    case 1: return launch_t<DT, 1, FINAL>(a, stream);
    case 2: return launch_t<DT, 2, FINAL>(a, stream);
    case 4: return launch_t<DT, 4, FINAL>(a, stream);
    case 8: return launch_t<DT, 8, FINAL>(a, stream);
    case 16: return launch_t<DT, 16, FINAL>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a) {
  return (a.dtype == PA_F16 || a.dtype == PA_BF16) && a.head_size == 128 &&
         query_vectors(a) <= 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const bool fin = a.partition_size == 0;
  if (a.dtype == PA_BF16)
    return fin ? dispatch_g<PA_BF16, true>(a, stream) : dispatch_g<PA_BF16, false>(a, stream);
  return fin ? dispatch_g<PA_F16, true>(a, stream) : dispatch_g<PA_F16, false>(a, stream);
}

}  // namespace pa
