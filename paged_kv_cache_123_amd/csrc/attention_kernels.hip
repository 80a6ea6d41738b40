// Paged decode attention for gfx950: single pass, split-K partition, reduce.
//
// What is computed ([VLLBC] walk-through of paper sections 4.1-4.2; [PUFANYI]
// "按 Block 分配" and its closing section; [DEEPSONAR] section 2.1 for GQA):
// for each sequence s and query head h, the new query q is scored against
// every cached key of KV head g = h / G, read block by block through the
// block table; softmax over the scores weights the cached values.
//
// Work decomposition (CDNA4, wave64):
//   * One workgroup of NW waves per (sequence, KV head, partition).  It serves
//     all G query heads of the KV head, so every K/V byte is read once.
//   * A tile is 16 consecutive logical tokens.  Each token's head_size row is
//     spread over LPT = D / VEC lanes, each lane owning one 16-byte vector
//     (VEC elements), so one wave-wide load covers TPL = 64 / LPT tokens and a
//     tile takes U = 16 / TPL loads per cache: whole 1-4 KiB contiguous runs.
//   * Waves take tiles round-robin; the next tile's K/V loads are issued
//     before the current tile is consumed (register double buffering).
//   * Scores: per-lane partial dot product (v_dot2 for 16-bit storage), then
//     an LPT-lane butterfly sum with DPP.  Each lane group (the LPT lanes of a
//     token) keeps its own online-softmax state (m, l, acc) in the log2
//     domain, so the main loop has no cross-lane max/sum traffic; lane groups
//     are merged with shuffles at the end and waves through LDS, in a fixed
//     order that depends only on logical positions (results are bit-identical
//     under any permutation of physical blocks).
//   * The block-table entries of a chunk of up to 2048 tokens are staged in
//     LDS once per workgroup.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "decode_common.h"
#include "launch.h"
#include "pagedkv.h"

#ifndef PA_VALU_OCCUPANCY
#define PA_VALU_OCCUPANCY
#endif
#ifndef PA_VALU_PIPELINE_BARRIER
#define PA_VALU_PIPELINE_BARRIER 1
#endif

namespace pa {
namespace {

using namespace dev;

// ---- the decode kernel ------------------------------------------------------
// FINAL: write the outputs in storage dtype (single pass); otherwise write the
// partition's (m, l, o) to the split workspace.
//
// A workgroup serves NQ query vectors that share the KV head: vector v is new
// token v >> log2_group of the sequence (one token per sequence when q_start is
// null, the decode case) and query head kvh * G + (v & (G - 1)), G = 1 <<
// log2_group.  Vector v sees the keys below bound[v] = L - n + (v >> log2_group)
// + 1 for a sequence with n new tokens; vectors past the sequence's new tokens
// see none and are not stored.  With a sliding window W > 0 it sees only the
// last W of them, positions from bound[v] - W on: reading starts at the first
// vector's window, and a partition wholly before it has no work.
template <int DT, int D, int NQ, int NW, bool FINAL>
__global__ __launch_bounds__(NW * 64) PA_VALU_OCCUPANCY void paged_decode_kernel(
    void* __restrict__ out, const void* __restrict__ query, const void* key_cache,
    const void* value_cache, const int32_t* __restrict__ block_tables,
    int64_t bt_stride, const int32_t* __restrict__ context_lens, int32_t num_heads,
    int32_t num_kv_heads, int32_t log2_block, int32_t partition_size, int32_t num_partitions,
    float scale_log2, float* __restrict__ ws_max, float* __restrict__ ws_sum,
    float* __restrict__ ws_out, const int2* __restrict__ items, AppendArgs ap,
    const int32_t* __restrict__ shared_blocks, int32_t log2_group,
    const int32_t* __restrict__ q_start, int32_t window) {
  using S = St<DT>;
  constexpr int VEC = S::VEC;
  constexpr int LPT = D / VEC;    // lanes per token
  constexpr int TPL = 64 / LPT;   // tokens per wave-wide load
  constexpr int U = kTile / TPL;  // loads per tile per cache
  static_assert(LPT >= 8 && LPT <= 32 && U >= 1, "unsupported head size");

  const WorkUnit wu = work_unit(items, num_kv_heads, FINAL ? 1 : num_partitions);
  const int p = wu.p;
  const int kvh = wu.kvh;
  const int s = wu.s;
  const int L = context_lens[s];
  const int t_begin = FINAL ? 0 : p * partition_size;
  if (t_begin >= L) return;  // empty partition: the reduce never reads it
  const int t_end = FINAL ? L : min(L, t_begin + partition_size);
  const int qlen = q_start ? q_start[s + 1] - q_start[s] : 1;
  // first key any vector of this sequence sees (the first new token's window)
  const int lo_min = window > 0 ? max(0, L - qlen + 1 - window) : 0;
  if (t_end <= lo_min) return;  // wholly before the window: the merge skips it

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lg = lane / LPT;   // lane group = token within a load
  const int sub = lane % LPT;  // which 16-byte vector of the row
  const int B = 1 << log2_block;
  // strides in 16-byte vectors: a block is [H_kv][B][D], a token row D / VEC
  const int64_t blk_stride_v = static_cast<int64_t>(num_kv_heads) * B * LPT;
  const int64_t head_off_v = static_cast<int64_t>(kvh) * B * LPT + sub;
  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * bt_stride;
  // tokens of the leading blocks other sequences share (cached loads)
  const int shared_tokens = shared_blocks ? (shared_blocks[s] << log2_block) : 0;
  if (ap.qsl) {
    apply_appends<LPT, NW * 64>(ap, s, kvh, L, t_begin, t_end, bt_row, log2_block,
                                static_cast<int64_t>(num_kv_heads) * (1 << log2_block) * LPT,
                                static_cast<int64_t>(kvh) * (1 << log2_block) * LPT);
    __syncthreads();  // the rows written above are read by other waves below
  }
  const int32_t h0 = kvh << log2_group;
  const int gmask = (1 << log2_group) - 1;
  const int64_t qrow0 = q_start ? q_start[s] : s;

  typename S::QReg q[NQ];
  int bound[NQ], lo[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int qi = j >> log2_group;
    bound[j] = qi < qlen ? L - qlen + qi + 1 : 0;
    lo[j] = window > 0 ? max(0, bound[j] - window) : 0;
    q[j] = S::zero_q();
    if (qi < qlen)
      q[j] = S::load_q(query, ((qrow0 + qi) * num_heads + h0 + (j & gmask)) * D + sub * VEC);
  }

  float m[NQ], l[NQ], acc[NQ][VEC];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[j][e] = 0.0f;
  }

  __shared__ int32_t sm_bt[kChunkTokens];
  const uint4* kc = static_cast<const uint4*>(key_cache);
  const uint4* vc = static_cast<const uint4*>(value_cache);

  for (int c0 = max(t_begin, lo_min); c0 < t_end; c0 += kChunkTokens) {
    const int c1 = min(c0 + kChunkTokens, t_end);
    const int b0 = c0 >> log2_block;
    const int nb = ((c1 - 1) >> log2_block) - b0 + 1;
    for (int i = threadIdx.x; i < nb; i += NW * 64) sm_bt[i] = bt_row[b0 + i];
    __syncthreads();

    const int ntiles = (c1 - c0 + kTile - 1) / kTile;
    // index (in 16-byte vectors) of this lane's part of token t, which is
    // clamped into the chunk so that tail lanes read a real, finite row
    auto vec_index = [&](int t) -> int64_t {
      const int tc = min(t, c1 - 1);
      const int32_t phys = sm_bt[(tc >> log2_block) - b0];
      const int off = tc & (B - 1);
      return static_cast<int64_t>(phys) * blk_stride_v + head_off_v + off * LPT;
    };

    // Tile i covers tokens c0 + 16 i ..; wave w takes tiles w, w + NW, ...
    auto load_tile = [&](auto kind, int i, uint4 (&kd)[U], uint4 (&vd)[U]) {
      constexpr bool NT = decltype(kind)::streaming;
      const int t0 = c0 + i * kTile;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t idx = vec_index(t0 + u * TPL + lg);
        kd[u] = load_kv<NT>(kc + idx);
        vd[u] = load_kv<NT>(vc + idx);
      }
    };
    auto consume = [&](int i, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
      const int t0 = c0 + i * kTile;
      // scores of this lane group's U tokens for all NQ vectors (log2 domain)
      float x[NQ][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * TPL + lg;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          const float d = group_sum<LPT>(S::dot(q[j], kr[u]));
          x[j][u] = (t < c1 && t < bound[j] && t >= lo[j]) ? d * scale_log2 : -INFINITY;
        }
      }
      // new running maximum of every vector; rescale what it has so far
      float ms[NQ];
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        float mt = m[j];
#pragma unroll
        for (int u = 0; u < U; ++u) mt = fmaxf(mt, x[j][u]);
        ms[j] = mt == -INFINITY ? 0.0f : mt;
        const float c = __builtin_amdgcn_exp2f(m[j] - ms[j]);
        l[j] *= c;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][e] *= c;
        m[j] = mt;
      }
      // accumulate token by token: one V row piece is converted at a time,
      // which keeps the live registers (and so the occupancy) down
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[VEC];
        S::to_float(vr[u], vf);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          const float pr = __builtin_amdgcn_exp2f(x[j][u] - ms[j]);
          l[j] += pr;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][e] = fmaf(pr, vf[e], acc[j][e]);
        }
      }
    };
    // A wave's tiles of one load kind, through a ring of kPrefetch + 1
    // register slots: tile k + kPrefetch is requested before tile k is
    // consumed.  The steady-state loop requests unconditionally, so the wait
    // before each consume leaves the prefetched loads in flight; the last
    // tiles drain without prefetch.
    constexpr int NBUF = kPrefetch + 1;
    auto run = [&](auto kind, int lo, int hi) {
      int first, my;
      wave_tiles(lo, hi, wave, NW, first, my);
      uint4 kb[NBUF][U], vb[NBUF][U];
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j)
        if (j < my) load_tile(kind, first + j * NW, kb[j], vb[j]);
      int k = 0;
      for (; k + NBUF - 1 + kPrefetch < my; k += NBUF) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          load_tile(kind, first + (k + j + kPrefetch) * NW, kb[(j + kPrefetch) % NBUF],
                    vb[(j + kPrefetch) % NBUF]);
#if PA_VALU_PIPELINE_BARRIER
          // keep the scheduler from sinking these loads below the consume
          __builtin_amdgcn_sched_barrier(0);
#endif
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
    // Tiles that start below shared_tokens read shared blocks: cached loads;
    // the rest stream.  Each wave still takes its tiles in index order.
    // Measured choice of loop: the two-kind pipeline for one bf16 or fp32
    // query vector (long context 2600 vs 2654 us); for fp16 it needs 128+
    // VGPRs and loses to the single loop below, which keeps 4 waves per SIMD
    // (Llama-7B 186.2 vs 185.5 us); several query vectors would spill in it.
    if constexpr (NQ == 1 && DT != PA_F16) {
      const int n_cached = min(ntiles, max(0, (shared_tokens - c0 + kTile - 1) / kTile));
      run(LoadKind<false>{}, 0, n_cached);
      run(LoadKind<true>{}, n_cached, ntiles);
    } else {
      // one loop with the load kind chosen per tile
      const int my_tiles = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;
      auto load_any = [&](int it, uint4 (&kd)[U], uint4 (&vd)[U]) {
        const int i = wave + it * NW;
        if (c0 + i * kTile >= shared_tokens) load_tile(LoadKind<true>{}, i, kd, vd);
        else load_tile(LoadKind<false>{}, i, kd, vd);
      };
      uint4 kb[NBUF][U], vb[NBUF][U];
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j)
        if (j < my_tiles) load_any(j, kb[j], vb[j]);
      for (int it = 0; it < my_tiles; it += NBUF) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          if (it + j < my_tiles) {
            if (it + j + kPrefetch < my_tiles)
              load_any(it + j + kPrefetch, kb[(j + kPrefetch) % NBUF], vb[(j + kPrefetch) % NBUF]);
            consume(wave + (it + j) * NW, kb[j], vb[j]);
          }
        }
      }
    }
    __syncthreads();  // sm_bt is rewritten by the next chunk
  }

  // ---- merge the lane groups of this wave (lanes sharing `sub`) ----
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const float mo = __shfl_xor(m[j], off);
      const float lo = __shfl_xor(l[j], off);
      const float mt = fmaxf(m[j], mo);
      const float ms = mt == -INFINITY ? 0.0f : mt;
      const float ca = __builtin_amdgcn_exp2f(m[j] - ms);
      const float cb = __builtin_amdgcn_exp2f(mo - ms);
      // a + b == b + a exactly, so both partner lanes end with the same value
      l[j] = l[j] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = __shfl_xor(acc[j][e], off);
        acc[j][e] = acc[j][e] * ca + ao * cb;
      }
      m[j] = mt;
    }
  }

  // ---- merge the waves through LDS, in wave order ----
  __shared__ float sm_m[NW][NQ];
  __shared__ float sm_l[NW][NQ];
  __shared__ float sm_acc[NW][NQ][D];
  if (lg == 0) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[wave][j][sub * VEC + e] = acc[j][e];
      if (sub == 0) {
        sm_m[wave][j] = m[j];
        sm_l[wave][j] = l[j];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NQ * D; i += NW * 64) {
    const int j = i / D, d = i % D;
    const int qi = j >> log2_group;
    if (qi >= qlen) continue;  // a vector past this sequence's new tokens
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][j]);
    const float Ms = M == -INFINITY ? 0.0f : M;  // no visible key in this range
    float lsum = 0.0f, a = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = __builtin_amdgcn_exp2f(sm_m[w][j] - Ms);  // idle wave: exp2(-inf) = 0
      lsum = fmaf(sm_l[w][j], c, lsum);
      a = fmaf(sm_acc[w][j][d], c, a);
    }
    const int64_t row = (qrow0 + qi) * num_heads + h0 + (j & gmask);
    if constexpr (FINAL) {
      S::store(out, row * D + d, a / lsum);
    } else {
      const int64_t slot = row * num_partitions + p;
      ws_out[slot * D + d] = lsum > 0.0f ? a / lsum : 0.0f;  // empty range: weight 0
      if (d == 0) {
        ws_max[slot] = M * kLn2;
        ws_sum[slot] = lsum;
      }
    }
  }
}

// Merge of the parts of one (row, head): M = max m_p, a_p = l_p exp(m_p - M),
// out = sum a_p o_p / sum a_p.  The parts are the partitions of a split
// launch, or the ranks of a context-parallel group.
//
// One wave per (row, head), four heads per workgroup, nothing shared between
// waves.  Parts are taken in chunks of 64: lane i loads m and l of part
// c0 + i, the wave reduces the maximum and the weight sum with shuffles, and
// each lane accumulates its D/64 dims of o over the chunk, the weight of part
// p read from lane p.  The o loads do not depend on the weights, so the first
// kMergeBatch of them are issued before the weights are computed; a load
// past the chunk's last part re-reads that part and gets weight 0.  A later
// chunk rescales what was accumulated when the maximum grows.  A part with
// l_p = 0 (no visible key) has weight 0; a row with no key at all merges to
// m = -inf, l = 0, o = 0.
constexpr int kMergeBatch = 16;

template <int D>
__device__ __forceinline__ void load_parts(float (&v)[kMergeBatch][D / 64], const float* o,
                                           int64_t part_o, int i, int cn) {
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    const float* q = o + static_cast<int64_t>(min(i + k, cn - 1)) * part_o;
    if constexpr (D == 128) {
      const float2 t = *reinterpret_cast<const float2*>(q);
      v[k][0] = t.x;
      v[k][1] = t.y;
    } else {
      v[k][0] = *q;
    }
  }
}

template <int DT, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeDst dst, PartView src,
                                                    const int32_t* __restrict__ context_lens,
                                                    int32_t num_heads, int32_t partition_size,
                                                    int32_t num_parts,
                                                    const int32_t* __restrict__ q_start,
                                                    int32_t window) {
  constexpr int DPL = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int head_groups = (num_heads + 3) / 4;  // four heads (waves) per workgroup
  const int h = static_cast<int>(blockIdx.x % head_groups) * 4 + (threadIdx.x >> 6);
  const int s = static_cast<int>(blockIdx.x / head_groups);
  if (h >= num_heads) return;  // no barrier below
  // split launches: only the partitions below the sequence's length exist
  const int L = context_lens ? context_lens[s] : 0;
  const int np = context_lens ? min((L + partition_size - 1) / partition_size, num_parts)
                              : num_parts;
  // one output row per new token of the sequence (one row when q_start is
  // null); workgroup y of the launch takes tokens y, y + gridDim.y, ...
  const int qlen = q_start ? q_start[s + 1] - q_start[s] : 1;
  const int64_t qrow0 = q_start ? q_start[s] : s;
  for (int qi = static_cast<int>(blockIdx.y); qi < qlen; qi += static_cast<int>(gridDim.y)) {
    const int64_t row = (qrow0 + qi) * num_heads + h;
    // with a sliding window, partitions before this row's window hold nothing
    const int p0 = window > 0 ? max(0, L - qlen + qi + 1 - window) / partition_size : 0;
    const float* mrow = src.m + row * src.row_ml;
    const float* lrow = src.l + row * src.row_ml;
    const float* orow = src.o + row * src.row_o + lane * DPL;
    float M = -INFINITY, wsum = 0.0f;
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.0f;
    for (int c0 = p0; c0 < np; c0 += 64) {
      const int cn = min(64, np - c0);
      const float* o = orow + static_cast<int64_t>(c0) * src.part_o;
      float v[kMergeBatch][DPL];
      load_parts<D>(v, o, src.part_o, 0, cn);
      const int64_t k = static_cast<int64_t>(c0 + min(lane, cn - 1)) * src.part_ml;
      const float mv = lane < cn ? mrow[k] : -INFINITY;
      const float lv = lane < cn ? lrow[k] : 0.0f;
      float mc = mv;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mc = fmaxf(mc, __shfl_xor(mc, off));
      const float Mn = fmaxf(M, mc);
      const float Ms = Mn == -INFINITY ? 0.0f : Mn;
      // rescale the earlier chunks (nothing to rescale before the first)
      const float corr = M == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((M - Ms) * kLog2e);
      M = Mn;
      const float w = lv * __builtin_amdgcn_exp2f((mv - Ms) * kLog2e);
      float ws = w;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off);
      wsum = wsum * corr + ws;
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[j] *= corr;
      for (int i = 0;;) {
#pragma unroll
        for (int kk = 0; kk < kMergeBatch; ++kk) {
          const float wk = i + kk < cn ? __shfl(w, i + kk) : 0.0f;
#pragma unroll
          for (int j = 0; j < DPL; ++j) acc[j] = fmaf(wk, v[kk][j], acc[j]);
        }
        i += kMergeBatch;
        if (i >= cn) break;
        load_parts<D>(v, o, src.part_o, i, cn);
      }
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      const float merged = wsum > 0.0f ? acc[j] / wsum : 0.0f;
      const int64_t e = row * D + lane * DPL + j;
      if (dst.out)
        St<DT>::store(dst.out, e, merged);
      else
        dst.o[e] = merged;
    }
    if (!dst.out && lane == 0) {
      dst.m[row] = M;
      dst.l[row] = wsum;
    }
  }
}

template <int DT, int D, int NQ, bool FINAL, int NW>
hipError_t launch_decode_nw(const DecodeArgs& a, hipStream_t stream) {
  int log2_block = 0;
  while ((1 << log2_block) < a.block_size) ++log2_block;
  int log2_group = 0;
  while ((1 << log2_group) < a.num_heads / a.num_kv_heads) ++log2_group;
  const dim3 grid = a.items ? dim3(static_cast<uint32_t>(a.num_items * a.num_kv_heads))
                            : dim3(static_cast<uint32_t>((FINAL ? 1 : a.num_partitions) *
                                                         static_cast<int64_t>(a.num_kv_heads) *
                                                         a.num_seqs));
  hipLaunchKernelGGL((paged_decode_kernel<DT, D, NQ, NW, FINAL>), grid, dim3(NW * 64), 0, stream,
                     a.out, a.query, a.key_cache, a.value_cache, a.block_tables, a.bt_stride,
                     a.context_lens, a.num_heads, a.num_kv_heads, log2_block, a.partition_size,
                     a.num_partitions, a.scale * kLog2e, a.ws_max, a.ws_sum, a.ws_out,
                     reinterpret_cast<const int2*>(a.items), a.append,
                     a.shared_blocks, log2_group, a.q_start, a.window);
  return hipGetLastError();
}

template <int DT, int D, int NQ, bool FINAL>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  // many query vectors of a wide head need more registers than 8-wave
  // workgroups leave each wave: those keep the shared-case wave count
  constexpr int kWaves = NQ * D > 512 ? PA_VALU_WAVES_SHARED : PA_VALU_WAVES;
  return a.shared_blocks ? launch_decode_nw<DT, D, NQ, FINAL, PA_VALU_WAVES_SHARED>(a, stream)
                         : launch_decode_nw<DT, D, NQ, FINAL, kWaves>(a, stream);
}

template <int DT, int D, bool FINAL>
hipError_t dispatch_g(const DecodeArgs& a, hipStream_t stream) {
  switch (query_vectors(a)) {
    case 1: return launch_decode_t<DT, D, 1, FINAL>(a, stream);
    case 2: return launch_decode_t<DT, D, 2, FINAL>(a, stream);
    case 4: return launch_decode_t<DT, D, 4, FINAL>(a, stream);
    case 8: return launch_decode_t<DT, D, 8, FINAL>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool FINAL>
hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t stream) {
  const bool d64 = a.head_size == 64;
  switch (a.dtype) {
    case PA_F32:
      return d64 ? dispatch_g<PA_F32, 64, FINAL>(a, stream)
                 : dispatch_g<PA_F32, 128, FINAL>(a, stream);
    case PA_F16:
      return d64 ? dispatch_g<PA_F16, 64, FINAL>(a, stream)
                 : dispatch_g<PA_F16, 128, FINAL>(a, stream);
    case PA_BF16:
      return d64 ? dispatch_g<PA_BF16, 64, FINAL>(a, stream)
                 : dispatch_g<PA_BF16, 128, FINAL>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_merge_t(const MergeDst& dst, const PartView& src, const int32_t* context_lens,
                          int32_t num_rows, int32_t num_heads, int32_t partition_size,
                          int32_t num_parts, const int32_t* q_start, int32_t window,
                          int32_t token_split, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>((num_heads + 3) / 4) * num_rows;
  hipLaunchKernelGGL((merge_kernel<DT, D>),
                     dim3(static_cast<uint32_t>(grid), static_cast<uint32_t>(token_split)),
                     dim3(256), 0, stream, dst, src, context_lens, num_heads, partition_size,
                     num_parts, q_start, window);
  return hipGetLastError();
}

hipError_t launch_merge(int32_t dtype, int32_t head_size, const MergeDst& dst,
                        const PartView& src, const int32_t* context_lens, int32_t num_rows,
                        int32_t num_heads, int32_t partition_size, int32_t num_parts,
                        const int32_t* q_start, int32_t window, hipStream_t stream,
                        int32_t token_split = 1) {
  const bool d64 = head_size == 64;
#define PA_MERGE(DT)                                                                     \
  return d64 ? launch_merge_t<DT, 64>(dst, src, context_lens, num_rows, num_heads,       \
                                      partition_size, num_parts, q_start, window,        \
                                      token_split, stream)                               \
             : launch_merge_t<DT, 128>(dst, src, context_lens, num_rows, num_heads,      \
                                       partition_size, num_parts, q_start, window,       \
                                       token_split, stream)
  switch (dtype) {
    case PA_F32: PA_MERGE(PA_F32);
    case PA_F16: PA_MERGE(PA_F16);
    case PA_BF16: PA_MERGE(PA_BF16);
    default: return hipErrorInvalidValue;
  }
#undef PA_MERGE
}

// the split workspace as parts: [row][NP] for m and l, [row][NP][D] for o
PartView split_parts(const DecodeArgs& a) {
  return PartView{a.ws_max, a.ws_sum, a.ws_out, 1, a.num_partitions,
                  a.head_size, static_cast<int64_t>(a.num_partitions) * a.head_size};
}

}  // namespace

namespace {
// 0: automatic, 1: vector kernel, 2: matrix-core kernel where supported.
// Starts from PAGEDKV_DECODE_KERNEL=valu|mfma if set.
std::atomic<int> g_decode_kernel{-1};

int decode_kernel_mode() {
  int mode = g_decode_kernel.load(std::memory_order_relaxed);
  if (mode < 0) {
    const char* v = std::getenv("PAGEDKV_DECODE_KERNEL");
    mode = !v ? 0 : std::strcmp(v, "valu") == 0 ? 1 : std::strcmp(v, "mfma") == 0 ? 2 : 0;
    int expected = -1;
    g_decode_kernel.compare_exchange_strong(expected, mode);
    mode = g_decode_kernel.load(std::memory_order_relaxed);
  }
  return mode;
}
}  // namespace

int set_decode_kernel(int mode) {
  const int prev = decode_kernel_mode();
  g_decode_kernel.store(mode, std::memory_order_relaxed);
  return prev;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int mode = decode_kernel_mode();
  const int nq = query_vectors(a);
  const bool can_mfma = decode_mfma_supported(a);
  // group items (cascade plans) exist only in the matrix-core kernels: the
  // partition kernel, or the single-pass cascade kernel
  if (a.max_group > 0) {
    if (!can_mfma) return hipErrorInvalidValue;
    return a.partition_size == 0 || a.cascade_chunked ? launch_cascade_single(a, stream)
                                                      : launch_decode_mfma(a, stream);
  }
  const bool can_valu = nq <= 8;
  // automatic: matrix cores as soon as a workgroup serves several query vectors
  const bool mfma = mode == 1 ? (!can_valu && can_mfma)
                  : mode == 2 ? can_mfma
                              : (can_mfma && nq >= 2);
  if (mfma) return launch_decode_mfma(a, stream);
  if (!can_valu) return hipErrorInvalidValue;
  return a.partition_size == 0 ? dispatch_decode<true>(a, stream)
                               : dispatch_decode<false>(a, stream);
}

hipError_t launch_split_reduce(const DecodeArgs& a, hipStream_t stream) {
  return launch_merge(a.dtype, a.head_size, MergeDst{a.out, nullptr, nullptr, nullptr},
                      split_parts(a), a.context_lens, a.num_seqs, a.num_heads, a.partition_size,
                      a.num_partitions, a.q_start, a.window, stream, a.merge_token_split);
}

hipError_t launch_split_reduce_partials(const DecodeArgs& a, float* m, float* l, float* o,
                                        hipStream_t stream) {
  return launch_merge(a.dtype, a.head_size, MergeDst{nullptr, m, l, o}, split_parts(a),
                      a.context_lens, a.num_seqs, a.num_heads, a.partition_size,
                      a.num_partitions, a.q_start, a.window, stream);
}

hipError_t launch_merge_ranks(void* out, const float* m, const float* l, const float* o,
                              int32_t num_parts, int32_t num_seqs, int32_t num_heads,
                              int32_t head_size, int32_t dtype, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads;
  return launch_merge(dtype, head_size, MergeDst{out, nullptr, nullptr, nullptr},
                      PartView{m, l, o, rows, 1, rows * head_size, head_size}, nullptr,
                      num_seqs, num_heads, 1, num_parts, nullptr, 0, stream);
}

}  // namespace pa
