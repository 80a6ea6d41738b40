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
#include "status.h"

#ifndef PA_MFMA_OCCUPANCY
#define PA_MFMA_OCCUPANCY
#endif

// Per-workgroup timeline of the single-pass cascade kernel, compiled in only
// with PA_TIMELINE=1 (a diagnostic build): workgroup i < kTimelineMax
// records the real-time counter (100 MHz) at entry, when its first round of
// tiles is described, and at exit, and the hardware ids of the CU it ran on.
#ifndef PA_TIMELINE
#define PA_TIMELINE 0
#endif

namespace pa {

constexpr int64_t kTimelineMax = 8192;
#if PA_TIMELINE
__device__ uint64_t g_timeline[kTimelineMax * 4];
#endif

namespace {

using namespace dev;


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
  static_assert(NQ >= 1 && NQ <= 16, "query vectors must fit the 16 MFMA columns");

  const WorkUnit wu = work_unit(items, num_kv_heads, FINAL ? 1 : num_partitions);
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
  if (ap.qsl && !gmem) {
    apply_appends<DV, NW * 64>(ap, s, kvh, L, t_begin, t_end, bt_row, log2_block,
                                static_cast<int64_t>(num_kv_heads) * (1 << log2_block) * DV,
                                static_cast<int64_t>(kvh) * (1 << log2_block) * DV);
    __syncthreads();  // the rows written above are read by other waves below
  }
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
      bool vis[4];  // tokens grp + 4j for head col
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + grp + 4 * j;
        vis[j] = (t < c1) & (t < bound) & (t >= lo);  // no short-circuit: selects, not branches
      }
      mfma_tile_update<DT>(kr, vr, qv, vis, scale_log2, m, lsum, o);
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
                            : dim3(static_cast<uint32_t>((FINAL ? 1 : a.num_partitions) *
                                                         static_cast<int64_t>(a.num_kv_heads) *
                                                         a.num_seqs));
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

// ---- single-pass cascade ----------------------------------------------------
// One workgroup per (item, KV head) of a single-pass cascade plan.  A group
// item (s < 0) serves the members of chunk -1 - s of the plan's group section
// (column c holds member c >> log2_group's query): it reads the prefix of
// it.y tokens once through the first member's table with every member's
// columns live, then each member's own tokens [prefix, L_m) through that
// member's table with only that member's columns live, and stores every
// member's output.  An item (s, 0) reads sequence s alone.
//
// The step's cache writes of every member ride on the attention's loads:
// tiles that hold a member's new tokens take those rows from key/value, and
// the old slots of a copy-on-write tail from the source block; every lane
// then stores what it loaded to the cache slot the row belongs to (and the
// new tokens' slots).  No workgroup reads a row written during the launch,
// so the writes need no barrier and cost no extra loads.
//
// Tokens go in rounds of at most kChunkTokens.  A round is a list of pieces
// (a run of the prefix or of one member's own tokens); thread 0 lists them,
// then the workgroup stages their table entries in LDS and describes their
// 16-token tiles (owner, first token, piece end, table base), and the waves
// take the round's tiles round-robin.  Tile boundaries depend only on logical
// positions, so the result does not depend on where the blocks lie.
#ifndef PA_CASCADE_PREFETCH
#define PA_CASCADE_PREFETCH 1
#endif
constexpr int kCascadePrefetch = PA_CASCADE_PREFETCH;  // tiles in flight per wave
constexpr int kMaxMembers = 16;
constexpr int kMaxPieces = kMaxMembers + 1;
constexpr int kRoundTiles = kChunkTokens / kTile + kMaxPieces;

template <int DT, int NQ, int NW>
__global__ __launch_bounds__(NW * 64) PA_MFMA_OCCUPANCY void cascade_decode_kernel(
    void* __restrict__ out, const void* __restrict__ query, const void* key_cache,
    const void* value_cache, const int32_t* __restrict__ block_tables, int64_t bt_stride,
    const int32_t* __restrict__ context_lens, int32_t num_heads, int32_t num_kv_heads,
    int32_t log2_block, float scale_log2, const int2* __restrict__ items, int64_t num_items,
    AppendArgs ap, int32_t log2_group, int32_t partition_size, int32_t num_partitions,
    float* __restrict__ ws_max, float* __restrict__ ws_sum, float* __restrict__ ws_out) {
  constexpr int D = 128;
  constexpr int DV = D / 8;
  constexpr int NK = D / 32;
  constexpr int NE = 8;
  constexpr int U = 4;
  static_assert(NQ >= 1 && NQ <= 16, "query vectors must fit the 16 MFMA columns");

#if PA_TIMELINE
  const uint64_t tl_entry = __builtin_amdgcn_s_memrealtime();
  uint64_t tl_ready = 0;
#endif
  const int2 it = items[blockIdx.x / num_kv_heads];
  const int kvh = static_cast<int>(blockIdx.x % num_kv_heads);
  __shared__ int32_t sm_mem[kMaxMembers];  // members (batch rows)
  __shared__ int32_t sm_len[kMaxMembers];  // their context lengths
  // the step's writes per member: first new position (INT_MAX: none), first
  // position written (the copied tail's block start, or the first new
  // position), copy-on-write source block (-1: none), input row of p0
  __shared__ int32_t sm_p0[kMaxMembers];
  __shared__ int32_t sm_touch[kMaxMembers];
  __shared__ int32_t sm_cow[kMaxMembers];
  __shared__ int32_t sm_q0[kMaxMembers];
  // chunked plans (partition_size > 0) keep each chunk's prefix length after
  // the member offsets; single-pass plans carry it in the item
  const bool chunked = partition_size > 0;
  int nmem = 1;
  const int32_t* gm = nullptr;
  int prefix = 0;
  if (it.x < 0) {
    const int32_t* gsec = reinterpret_cast<const int32_t*>(items + num_items);
    const int nc = gsec[0];
    const int c = -1 - it.x;
    const int m0 = gsec[1 + c];
    nmem = min(gsec[2 + c] - m0, kMaxMembers);
    gm = gsec + 2 + nc + (chunked ? nc : 0) + m0;
    prefix = chunked ? gsec[2 + nc + c] : it.y;
  }
  if (static_cast<int>(threadIdx.x) < nmem) {
    const int32_t r = gm ? gm[threadIdx.x] : it.x;
    const int L = context_lens[r];
    int p0 = INT_MAX, touch = INT_MAX, cow = -1, q0 = 0;
    if (ap.qsl) {
      q0 = ap.qsl[r];
      const int n = ap.qsl[r + 1] - q0;
      if (n > 0) {
        p0 = L - n;
        touch = p0;
        if (ap.cow_src && ap.cow_src[r] >= 0) {
          cow = static_cast<int32_t>(ap.cow_src[r]);
          touch = (p0 >> log2_block) << log2_block;
        }
      }
    }
    sm_mem[threadIdx.x] = r;
    sm_len[threadIdx.x] = L;
    sm_p0[threadIdx.x] = p0;
    sm_touch[threadIdx.x] = touch;
    sm_cow[threadIdx.x] = cow;
    sm_q0[threadIdx.x] = q0;
  }
  __syncthreads();
  // What the item reads: a run [sa, sb) of the shared prefix with every
  // member's columns live, then (with_members) each member's own tokens
  // [ma, min(L_m, me)) with only that member's columns live.  out_part: the
  // slot of the partials it writes (chunked plans), or -1 for the output.
  //   single pass, group:  [0, prefix), then [prefix, L_m)
  //   single pass, alone:  [0, L)
  //   chunked, group j < prefix / P:  [jP, (j + 1)P) of the prefix, slot j
  //   chunked, group j = prefix / P:  [jP, prefix), then [prefix, L_m), slot j
  //   chunked, alone (s, p):  [pP, min((p + 1)P, L)), slot p
  int sa = 0, sb = 0, ma = 0, me = INT_MAX, out_part = -1;
  bool with_members = true;
  if (gm) {
    ma = prefix;
    sb = prefix;
    if (chunked) {
      const int pf = prefix / partition_size;
      out_part = it.y;
      sa = it.y * partition_size;
      if (it.y < pf) {
        sb = sa + partition_size;
        with_members = false;
      }
    }
  } else if (chunked) {
    out_part = it.y;
    ma = it.y * partition_size;
    me = ma + partition_size;
  }

  const int B = 1 << log2_block;
  const int64_t blk_stride_v = static_cast<int64_t>(num_kv_heads) * B * DV;
  const int64_t head_off_v = static_cast<int64_t>(kvh) * B * DV;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int h0 = kvh << log2_group;
  const int gmask = (1 << log2_group) - 1;
  const int my_m = col >> log2_group;  // member of this column
  const bool my_valid = col < NQ && my_m < nmem;
  const int64_t my_row = sm_mem[my_valid ? my_m : 0];

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

  __shared__ int32_t sm_bt[kChunkTokens + kMaxPieces];
  __shared__ int4 sm_piece[kMaxPieces];  // {first token, end, owner (-1: all), first entry}
  __shared__ int32_t sm_ptile[kMaxPieces + 1];  // first tile of each piece
  __shared__ int4 sm_tile[kRoundTiles];  // {owner, first token, piece end, table base}
  __shared__ int32_t sm_round[4];        // {pieces, next segment, next token, entries}
  const uint4* kc = static_cast<const uint4*>(key_cache);
  const uint4* vc = static_cast<const uint4*>(value_cache);
  const int k_tok = (col >> 2) + 4 * (col & 3);  // token of this lane's K row

  // segment g: the shared run (g == 0 when there is one), else a member's own tokens
  const bool has_shared = sb > sa;
  const int nseg = (has_shared ? 1 : 0) + (with_members ? nmem : 0);
  auto segment = [&](int g, int& a, int& b, int& owner) {
    if (has_shared && g == 0) {
      a = sa;
      b = sb;
      owner = -1;
    } else {
      owner = g - (has_shared ? 1 : 0);
      a = ma;
      b = min(sm_len[owner], me);
    }
  };
  auto table_row = [&](int owner) {
    return block_tables + static_cast<int64_t>(sm_mem[owner < 0 ? 0 : owner]) * bt_stride;
  };
  int seg = 0, pos = 0;
  {
    int a, b, ow;
    segment(0, a, b, ow);
    pos = a;
  }
  while (seg < nseg) {
    if (threadIdx.x == 0) {  // list this round's pieces
      int np = 0, tok = 0, ent = 0, tiles = 0, g = seg, q = pos;
      while (g < nseg && tok < kChunkTokens && np < kMaxPieces) {
        int a, b, ow;
        segment(g, a, b, ow);
        const int e = max(q, min(b, q + (kChunkTokens - tok)));
        sm_piece[np] = make_int4(q, e, ow, ent);
        sm_ptile[np] = tiles;
        if (e > q) {
          ent += ((e - 1) >> log2_block) - (q >> log2_block) + 1;
          tiles += (e - q + kTile - 1) / kTile;
          tok += e - q;
        }
        ++np;
        if (e >= b) {
          if (++g < nseg) segment(g, q, b, ow);
        } else {
          q = e;
        }
      }
      sm_ptile[np] = tiles;
      sm_round[0] = np;
      sm_round[1] = g;
      sm_round[2] = q;
      sm_round[3] = ent;
    }
    __syncthreads();
    const int np = sm_round[0];
    const int ntiles = sm_ptile[np];
    const int nent = sm_round[3];
    // table entries and tile descriptors of the round
    for (int i = threadIdx.x; i < nent; i += NW * 64) {
      int k = 0;  // the last non-empty piece whose entries start at or below i
      for (int j = 1; j < np; ++j)
        if (sm_piece[j].w <= i && sm_piece[j].y > sm_piece[j].x) k = j;
      const int4 pc = sm_piece[k];
      sm_bt[i] = table_row(pc.z)[(pc.x >> log2_block) + (i - pc.w)];
    }
    for (int i = threadIdx.x; i < ntiles; i += NW * 64) {
      int k = 0;  // the last non-empty piece whose tiles start at or below i
      for (int j = 1; j < np; ++j)
        if (sm_ptile[j] <= i && sm_ptile[j + 1] > sm_ptile[j]) k = j;
      const int4 pc = sm_piece[k];
      sm_tile[i] = make_int4(pc.z, pc.x + (i - sm_ptile[k]) * kTile, pc.y,
                             pc.w - (pc.x >> log2_block));
    }
    __syncthreads();

    auto vec_index = [&](const int4& d, int t, int vec) -> int64_t {
      const int tc = min(t, d.z - 1);  // tail lanes read a real row of the piece
      const int32_t phys = sm_bt[d.w + (tc >> log2_block)];
      const int off = tc & (B - 1);
      return static_cast<int64_t>(phys) * blk_stride_v + head_off_v + off * DV + vec;
    };
    // a tile of member tokens the step writes (new rows or a copied tail)
    auto writes_rows = [&](const int4& d) { return d.x >= 0 && d.y + kTile > sm_touch[d.x]; };
    // where token t of such a tile is read: its new row in key/value, the
    // copy-on-write source block, or the cache
    auto source = [&](const int4& d, int t, int vec, const uint4* cache, const uint4* rows,
                      int64_t row_stride) -> const uint4* {
      const int tc = min(t, d.z - 1);
      const int p0 = sm_p0[d.x];
      if (tc >= p0) return rows + (sm_q0[d.x] + (tc - p0)) * row_stride + kvh * DV + vec;
      if (sm_cow[d.x] >= 0 && (tc >> log2_block) == (p0 >> log2_block))
        return cache + static_cast<int64_t>(sm_cow[d.x]) * blk_stride_v + head_off_v +
               (tc & (B - 1)) * DV + vec;
      return cache + vec_index(d, t, vec);
    };
    // the cache slot of token t receives what the lane loaded for it, if the
    // step writes t (in this piece, at or past the first written position)
    auto store_row = [&](const int4& d, int t, int vec, const uint4& v, uint4* cache) {
      if (t < d.z && t >= sm_touch[d.x]) cache[vec_index(d, t, vec)] = v;
    };
    auto load_tile = [&](int i, uint4 (&kd)[NK], uint4 (&vd)[U]) {
      const int4 d = sm_tile[i];
      if (writes_rows(d)) {
        const uint4* kp = source(d, d.y + k_tok, grp, kc, ap.key, ap.key_stride_v);
#pragma unroll
        for (int k = 0; k < NK; ++k) kd[k] = load_cached(kp + k * 4);
#pragma unroll
        for (int u = 0; u < U; ++u)
          vd[u] = load_cached(source(d, d.y + grp + 4 * u, col, vc, ap.value, ap.value_stride_v));
        return;
      }
#pragma unroll
      for (int k = 0; k < NK; ++k) kd[k] = load_stream(kc + vec_index(d, d.y + k_tok, k * 4 + grp));
#pragma unroll
      for (int u = 0; u < U; ++u) vd[u] = load_stream(vc + vec_index(d, d.y + grp + 4 * u, col));
    };
    auto consume = [&](int i, const uint4 (&kr)[NK], const uint4 (&vr)[U]) {
      const int4 d = sm_tile[i];
      if (writes_rows(d)) {
        const int t = d.y + k_tok;
#pragma unroll
        for (int k = 0; k < NK; ++k) store_row(d, t, k * 4 + grp, kr[k], ap.key_cache);
#pragma unroll
        for (int u = 0; u < U; ++u) store_row(d, d.y + grp + 4 * u, col, vr[u], ap.value_cache);
        if (kvh == 0 && grp == 0 && ap.slot_mapping && t < d.z && t >= sm_p0[d.x]) {
          const int64_t phys = sm_bt[d.w + (t >> log2_block)];
          ap.slot_mapping[sm_q0[d.x] + (t - sm_p0[d.x])] = phys * B + (t & (B - 1));
        }
      }
      const bool live = my_valid && (d.x < 0 || d.x == my_m);
      bool vis[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) vis[j] = live & (d.y + grp + 4 * j < d.z);
      mfma_tile_update<DT>(kr, vr, qv, vis, scale_log2, m, lsum, o);
    };
#if PA_TIMELINE
    if (tl_ready == 0) tl_ready = __builtin_amdgcn_s_memrealtime();
#endif
    // this wave's tiles of the round through a ring of kCascadePrefetch + 1 slots
    constexpr int NBUF = kCascadePrefetch + 1;
    int first, my;
    wave_tiles(0, ntiles, wave, NW, first, my);
    uint4 kb[NBUF][NK], vb[NBUF][U];
#pragma unroll
    for (int j = 0; j < kCascadePrefetch; ++j)
      if (j < my) load_tile(first + j * NW, kb[j], vb[j]);
    int k = 0;
    for (; k + NBUF - 1 + kCascadePrefetch < my; k += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        load_tile(first + (k + j + kCascadePrefetch) * NW, kb[(j + kCascadePrefetch) % NBUF],
                  vb[(j + kCascadePrefetch) % NBUF]);
        __builtin_amdgcn_sched_barrier(0);
        consume(first + (k + j) * NW, kb[j], vb[j]);
      }
    }
    for (; k < my; k += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        if (k + j < my) {
          if (k + j + kCascadePrefetch < my)
            load_tile(first + (k + j + kCascadePrefetch) * NW, kb[(j + kCascadePrefetch) % NBUF],
                      vb[(j + kCascadePrefetch) % NBUF]);
          consume(first + (k + j) * NW, kb[j], vb[j]);
        }
      }
    }
    seg = sm_round[1];
    pos = sm_round[2];
    __syncthreads();  // the round's LDS is rewritten by the next one
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
    const int j = i / D, dd = i % D;
    const int qi = j >> log2_group;
    if (qi >= nmem) continue;  // a column past the members
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][j]);
    const float Ms = M == -INFINITY ? 0.0f : M;
    float l = 0.0f, a = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = __builtin_amdgcn_exp2f(sm_m[w][j] - Ms);
      l = fmaf(sm_l[w][j], c, l);
      a = fmaf(sm_acc[w][j][dd], c, a);
    }
    const int64_t row = static_cast<int64_t>(sm_mem[qi]) * num_heads + h0 + (j & gmask);
    if (out_part < 0) {
      St<DT>::store(out, row * D + dd, a / l);
    } else {
      const int64_t slot = row * num_partitions + out_part;
      ws_out[slot * D + dd] = l > 0.0f ? a / l : 0.0f;
      if (dd == 0) {
        ws_max[slot] = M * kLn2;
        ws_sum[slot] = l;
      }
    }
  }
  // A chunked group's last item read each member's tokens past the prefix,
  // which may reach into later slots: those hold nothing for the merge.
  if (out_part >= 0 && gm && with_members) {
    const int G = 1 << log2_group;
    for (int qi = 0; qi < nmem; ++qi) {
      const int np = (sm_len[qi] + partition_size - 1) / partition_size;
      const int n = (np - out_part - 1) * G * D;
      for (int i = threadIdx.x; i < n; i += NW * 64) {
        const int dd = i % D, part = out_part + 1 + (i / D) % (np - out_part - 1);
        const int hh = i / (D * (np - out_part - 1));
        const int64_t slot =
            (static_cast<int64_t>(sm_mem[qi]) * num_heads + h0 + hh) * num_partitions + part;
        ws_out[slot * D + dd] = 0.0f;
        if (dd == 0) {
          ws_max[slot] = -INFINITY;
          ws_sum[slot] = 0.0f;
        }
      }
    }
  }
#if PA_TIMELINE
  __syncthreads();
  if (threadIdx.x == 0 && blockIdx.x < kTimelineMax) {
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    uint64_t* rec = g_timeline + 4 * static_cast<int64_t>(blockIdx.x);
    rec[0] = tl_entry;
    rec[1] = tl_ready;
    rec[2] = __builtin_amdgcn_s_memrealtime();
    rec[3] = (static_cast<uint64_t>(xcc) << 32) | hw;
  }
#endif
}

template <int DT, int NQ>
hipError_t launch_cascade_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = PA_MFMA_WAVES;
  int log2_block = 0;
  while ((1 << log2_block) < a.block_size) ++log2_block;
  int log2_group = 0;
  while ((1 << log2_group) < a.num_heads / a.num_kv_heads) ++log2_group;
  hipLaunchKernelGGL((cascade_decode_kernel<DT, NQ, NW>),
                     dim3(static_cast<uint32_t>(a.num_items * a.num_kv_heads)), dim3(NW * 64), 0,
                     stream, a.out, a.query, a.key_cache, a.value_cache, a.block_tables,
                     a.bt_stride, a.context_lens, a.num_heads, a.num_kv_heads, log2_block,
                     a.scale * kLog2e, reinterpret_cast<const int2*>(a.items), a.num_items,
                     a.append, log2_group, a.cascade_chunked ? a.partition_size : 0,
                     a.num_partitions, a.ws_max, a.ws_sum, a.ws_out);
  return hipGetLastError();
}

template <int DT>
hipError_t dispatch_cascade(const DecodeArgs& a, hipStream_t stream) {
  switch (query_vectors(a)) {
    case 1: return launch_cascade_t<DT, 1>(a, stream);
    case 2: return launch_cascade_t<DT, 2>(a, stream);
    case 4: return launch_cascade_t<DT, 4>(a, stream);
    case 8: return launch_cascade_t<DT, 8>(a, stream);
    case 16: return launch_cascade_t<DT, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a) {
  return (a.dtype == PA_F16 || a.dtype == PA_BF16) && a.head_size == 128 &&
         query_vectors(a) <= 16;
}

hipError_t launch_cascade_single(const DecodeArgs& a, hipStream_t stream) {
  if (!a.items || a.num_items < 1 || (a.partition_size != 0) != a.cascade_chunked)
    return hipErrorInvalidValue;
  return a.dtype == PA_BF16 ? dispatch_cascade<PA_BF16>(a, stream)
                            : dispatch_cascade<PA_F16>(a, stream);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const bool fin = a.partition_size == 0;
  if (a.dtype == PA_BF16)
    return fin ? dispatch_g<PA_BF16, true>(a, stream) : dispatch_g<PA_BF16, false>(a, stream);
  return fin ? dispatch_g<PA_F16, true>(a, stream) : dispatch_g<PA_F16, false>(a, stream);
}

}  // namespace pa

extern "C" int32_t pa_timeline_reset(void* stream) {
#if PA_TIMELINE
  void* dev = nullptr;
  if (hipGetSymbolAddress(&dev, HIP_SYMBOL(pa::g_timeline)) != hipSuccess ||
      hipMemsetAsync(dev, 0, sizeof(uint64_t) * 4 * pa::kTimelineMax,
                     static_cast<hipStream_t>(stream)) != hipSuccess)
    return pa::fail(PA_ELAUNCH, "pa_timeline_reset: could not clear the records");
  return PA_OK;
#else
  (void)stream;
  return pa::fail(PA_EINVAL, "pa_timeline_reset: library built without PA_TIMELINE");
#endif
}

extern "C" int32_t pa_timeline_read(uint64_t* records, int64_t capacity, int64_t* num_records) {
  if (!records || !num_records || capacity < 1)
    return pa::fail(PA_EINVAL, "pa_timeline_read: bad argument");
#if PA_TIMELINE
  const int64_t n = capacity < pa::kTimelineMax ? capacity : pa::kTimelineMax;
  if (hipMemcpyFromSymbol(records, HIP_SYMBOL(pa::g_timeline), sizeof(uint64_t) * 4 * n, 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return pa::fail(PA_ELAUNCH, "pa_timeline_read: copy failed");
  int64_t k = 0;
  while (k < n && records[4 * k] != 0) ++k;
  *num_records = k;
  return PA_OK;
#else
  return pa::fail(PA_EINVAL, "pa_timeline_read: library built without PA_TIMELINE");
#endif
}
