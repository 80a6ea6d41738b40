// Paged attention for prefill chunks on the matrix cores: every new token of
// a sequence is a query, causal over the new tokens ([DEEPSONAR] section 2.5
// schedules prefill chunks like decode tokens; [CSDN] section 2.3 lays a
// step's tokens out by query_start_loc).  The result is that of
// pa_paged_attention_multi; only the work layout differs.
//
// The host cuts each sequence's new tokens into query blocks of 128/G tokens
// (pa_query_blocks): with G query heads per KV head, a block holds 128 query
// vectors (token, head).  One workgroup of four waves serves one (block, KV
// head); wave w owns query vectors 32w .. 32w+31, two groups of 16, the
// columns of its matrix-core tiles.  The workgroup walks the keys the block
// sees in tiles of 64 tokens, double-buffered in LDS, with the loads of the
// next tile in registers while one is computed, so each K/V row is read from
// memory once per 128 query vectors and from LDS once per 32.  Each operand
// fragment a wave reads from LDS feeds the MFMAs of both of its groups, and
// the fragments of the next MFMAs are read while the current ones run.
// Every wave sees every tile, keeps the online softmax of its own columns and
// writes its outputs itself: no merge across waves.
//
// K and V rows sit in LDS as stored, padded to 18 16-byte units: the 16-byte
// K fragments a wave reads for a score MFMA (16 rows, 4 units) and the
// transposing V reads (8 rows of half a wave) then fall into distinct banks,
// and a read moves 1 KB in 4 cycles (at 17 units the K reads took 8); the
// value MFMA's operand (8 keys of one dim per lane) comes from the
// transposing LDS read of 16-bit elements.
//
// With the step's cache writes in the same launch (pa_prefill_step), keys
// from a sequence's first new position on are read from the step's key/value
// rows and the old slots of a copied tail block from its source block, so no
// workgroup reads a slot the launch writes; each row stores its own tokens'
// rows to their slots as its tile loop loads them.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <type_traits>

#include "decode_common.h"
#include "launch.h"
#include "pagedkv.h"

namespace pa {
namespace {

using namespace dev;

constexpr int kPrefillWaves = 4;
constexpr int kPrefillGroups = 2;  // 16-column query groups per wave
constexpr int kPrefillTile = 64;   // key tokens per LDS tile

// Maximum over the four lane groups of a column (lanes 16 and 32 apart):
// each permlane swap trades rows of 16 lanes between its two results, so
// their maximum is that of the lane and its partner.
__device__ __forceinline__ float column_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef short lds_s4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) lds_s4_t* lds_s4_ptr;

// Transposing LDS read of 16-bit elements: in each group of 16 lanes, lane
// i gets element i % 4 of the 4-element pieces that lanes i / 4, i / 4 + 4,
// i / 4 + 8 and i / 4 + 12 address.  With lane 4 r + c pointing at row r,
// elements 4 c .. 4 c + 3 of a row-major tile, lane i receives the four rows'
// element i: a column.
__device__ __forceinline__ uint2 read_columns(const void* lds_addr) {
  const lds_s4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(lds_addr));
  return __builtin_bit_cast(uint2, x);
}

// BIG_B: blocks of at least 4 tokens, so that the four keys a thread moves
// per tile share one block.  APPEND: the step's cache writes ride in the
// launch (pa_prefill_step).  SPLIT: the workgroup of item (row, p) attends
// the keys of partition p, [p P, (p + 1) P), and writes each query vector's
// partial (m, l, o) to the split workspace for the merge kernel
// (pa_paged_attention_prefill_split; not with APPEND).
template <int DT, bool BIG_B, bool APPEND, bool SPLIT>
__global__ __launch_bounds__(kPrefillWaves * 64) void prefill_kernel(
    void* __restrict__ out, const void* __restrict__ query, const void* key_cache,
    const void* value_cache, const int32_t* __restrict__ block_tables, int64_t bt_stride,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_lens,
    const int32_t* __restrict__ row_qsl, const int32_t* __restrict__ work_items,
    int32_t num_rows, int32_t num_heads, int32_t num_kv_heads, int32_t log2_block,
    int32_t log2_group, float scale_log2, int32_t window, AppendArgs ap,
    int32_t partition_size, int32_t num_partitions, float* __restrict__ ws_max,
    float* __restrict__ ws_sum, float* __restrict__ ws_out) {
  static_assert(!(APPEND && SPLIT), "the step's writes go with single-pass launches");
  constexpr int NW = kPrefillWaves;
  constexpr int NT = NW * 64;
  constexpr int QG = kPrefillGroups;
  constexpr int D = 128;
  constexpr int DV = D / 8;        // 16-byte units per token row
  constexpr int NK = D / 32;       // score MFMAs per 16-token sub-tile and group
  constexpr int NE = 8;            // value MFMA chunks (16 dims each)
  constexpr int KT = kPrefillTile;
  constexpr int NS = KT / 16;      // score sub-tiles per tile
  constexpr int KROW = DV + 2;     // padded LDS rows, in 16-byte units
  constexpr int VROW = DV + 2;
  constexpr int PER = KT * DV / NT;  // keys of each cache a thread moves per tile
  constexpr int NP = NS / 2;       // value MFMAs (K = 32 keys) per tile and dim chunk
  static_assert(KT * DV == NT * PER && NS % 2 == 0 && NT % DV == 0, "tile shape");
  using MM = Mma<DT>;

  __shared__ uint4 sk[2][KT * KROW];
  __shared__ uint4 sv[2][KT * VROW];
  __shared__ int32_t sm_bt[kChunkTokens];

  // without a list, the last row first: the rows of a sequence run together,
  // its longest first
  const int item = static_cast<int>(blockIdx.x / num_kv_heads);
  const int r = work_items ? work_items[2 * item] : num_rows - 1 - item;
  const int part = SPLIT ? work_items[2 * item + 1] : 0;
  if (SPLIT && (part < 0 || part >= num_partitions)) return;  // outside the workspace
  const int kvh = static_cast<int>(blockIdx.x % num_kv_heads);
  const int s = row_seq[r];
  const int L = row_lens[r];
  const int q0 = row_qsl[r];
  const int qlen = row_qsl[r + 1] - q0;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int gmask = (1 << log2_group) - 1;
  // group g's column of this lane: query vector v[g], its token qi[g] within
  // the block and its head hq[g]; the keys it sees: [lo[g], bound[g])
  int qi[QG], hq[QG], bound[QG], lo[QG];
  bool valid[QG];
  // the keys every column of this wave sees, [wlo_max, whi_min) (empty when
  // a column has no query), and those some column sees, [wlo_min, whi_max)
  int whi_min = INT_MAX, wlo_max = 0, whi_max = 0, wlo_min = INT_MAX;
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int v = wave * (16 * QG) + g * 16 + col;
    qi[g] = v >> log2_group;
    valid[g] = qi[g] < qlen;
    hq[g] = (kvh << log2_group) + (v & gmask);
    bound[g] = valid[g] ? L - qlen + qi[g] + 1 : 0;
    lo[g] = !valid[g] ? INT_MAX : window > 0 ? max(0, bound[g] - window) : 0;
    whi_min = min(whi_min, bound[g]);
    wlo_max = max(wlo_max, valid[g] ? lo[g] : INT_MAX);
    whi_max = max(whi_max, bound[g]);
    wlo_min = min(wlo_min, lo[g]);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    whi_min = min(whi_min, __shfl_xor(whi_min, off));
    wlo_max = max(wlo_max, __shfl_xor(wlo_max, off));
    whi_max = max(whi_max, __shfl_xor(whi_max, off));
    wlo_min = min(wlo_min, __shfl_xor(wlo_min, off));
  }
  // the block's first visible key, rounded down to a multiple of 4 with
  // blocks of 4 or more keys (a key before it is masked and lies in its
  // block): a thread's four keys of a tile then share one block
  const int lo_first = window > 0 ? max(0, L - qlen + 1 - window) : 0;
  const int lo_min = BIG_B ? lo_first & ~(PER - 1) : lo_first;

  uint4 qv[QG][NK];
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      qv[g][k] = make_uint4(0, 0, 0, 0);
      if (valid[g])
        qv[g][k] = *reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(query) +
            (static_cast<int64_t>(q0 + qi[g]) * num_heads + hq[g]) * D + k * 32 + grp * 8);
    }
  // per column: the reference maximum m (-inf before the column's first
  // visible key) and the value subtracted, ms (m, or 0 while m is -inf);
  // all_set: every column of the wave has a reference (wave-uniform)
  f32x4 o[QG][NE];
  float m[QG], ms[QG], lsum[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
#pragma unroll
    for (int e = 0; e < NE; ++e) o[g][e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    m[g] = -INFINITY;
    ms[g] = 0.0f;
    lsum[g] = 0.0f;
  }
  bool all_set = false;

  // this thread's share of each tile's loads: keys 2 my_keys, 2 my_keys + 1,
  // dims 8 my_unit .. + 7
  const int my_unit = tid & 15, my_keys = tid >> 4;
  // where this lane's transposing value reads start (bytes into a buffer):
  // lane 4 a + c of lane group grp points at row 4 grp + a, dims 4 c .. + 3;
  // chunk e adds 32 e bytes, the second half of the 32 keys 16 rows
  const int v_read = (4 * grp + (col >> 2)) * VROW * 16 + 8 * (col & 3);

  const int B = 1 << log2_block;
  const int64_t blk_stride_v = static_cast<int64_t>(num_kv_heads) * B * DV;
  const int64_t head_off_v = static_cast<int64_t>(kvh) * B * DV;
  const int32_t* bt_row = block_tables + static_cast<int64_t>(s) * bt_stride;
  const uint4* kc = static_cast<const uint4*>(key_cache);
  const uint4* vc = static_cast<const uint4*>(value_cache);
  // this thread's unit of its KV head's rows: a cache row of block b, offset
  // o is at (b * H_kv * B + o) * DV units from these (block ids and the
  // block stride in units fit 32 bits: one 32 x 32 -> 64-bit product)
  const uint4* kc_my = kc + head_off_v + my_unit;
  const uint4* vc_my = vc + head_off_v + my_unit;
  const uint32_t blk_units = static_cast<uint32_t>(blk_stride_v);

  // The step's cache writes, in the same launch: no workgroup reads a slot
  // written here.  Keys from the sequence's first new position p0 on come
  // from the step's key/value rows, the old slots of a copied tail block
  // from its source block.  Each row stores the rows of its own tokens to
  // their slots as its tile loop loads them (and, for KV head 0, the slots
  // to the mapping at its end); the sequence's first row copies the old
  // slots here.
  int p0 = INT_MAX, seq_q0 = 0, special = INT_MAX;
  int64_t cow = -1;
  // this thread's unit of new row p0 and of slot 0 of the copied tail
  // block's source (strides below 2^31 units)
  const uint4 *key_new = nullptr, *value_new = nullptr, *key_cow = nullptr, *value_cow = nullptr;
  const uint32_t key_str = static_cast<uint32_t>(ap.key_stride_v);
  const uint32_t value_str = static_cast<uint32_t>(ap.value_stride_v);
  if (APPEND) {
    seq_q0 = ap.qsl[s];
    p0 = L - qlen - (q0 - seq_q0);
    key_new = ap.key + seq_q0 * ap.key_stride_v + kvh * DV + my_unit;
    value_new = ap.value + seq_q0 * ap.value_stride_v + kvh * DV + my_unit;
    cow = ap.cow_src ? ap.cow_src[s] : -1;
    key_cow = kc_my + max(cow, int64_t{0}) * blk_stride_v;
    value_cow = vc_my + max(cow, int64_t{0}) * blk_stride_v;
    special = cow >= 0 ? (p0 >> log2_block) << log2_block : p0;  // first key read elsewhere
    if (cow >= 0 && q0 == seq_q0) {
      const int jb = p0 >> log2_block;
      const int64_t from = cow * blk_stride_v + head_off_v;
      const int64_t to = static_cast<int64_t>(bt_row[jb]) * blk_stride_v + head_off_v;
      for (int i = tid; i < (p0 - (jb << log2_block)) * DV; i += NT) {
        ap.key_cache[to + i] = ap.key_cache[from + i];
        ap.value_cache[to + i] = ap.value_cache[from + i];
      }
    }
  }

  // keys [lo_min, L) in two ranges: the cache's rows of the tiles before
  // the first key read elsewhere (all of them without the step's writes),
  // then the rest, one copy of the loop per range (no branch on the range
  // in the pipeline).  The ranges meet on a tile boundary of the single
  // range: the same tiles, so the same arithmetic, as without the writes.
  const int split =
      APPEND ? lo_min + (max(min(special, L) - lo_min, 0) / KT) * KT : L;
  auto range = [&](auto phase_tag, int r_begin, int r_end) {
    constexpr bool phase = decltype(phase_tag)::value;
    for (int c0 = r_begin; c0 < r_end; c0 += kChunkTokens) {
      const int c1 = min(c0 + kChunkTokens, r_end);
      const int b0 = c0 >> log2_block;
      const int nb = ((c1 - 1) >> log2_block) - b0 + 1;
      for (int i = tid; i < nb; i += NT) sm_bt[i] = bt_row[b0 + i];
      __syncthreads();
      const int ntiles = (c1 - c0 + KT - 1) / KT;
      // rows of tile t into registers; rows past the chunk repeat its last
      // row, so tiles beyond the last are loaded too (unconditional loads
      // keep the wait counts of the pipeline static) and hit that one row.
      // The addresses first, then one load per key and cache (loads in
      // branches would leave the pipeline's waits to the compiler's most
      // cautious count).
      auto gload = [&](int t, uint4 (&pk)[PER], uint4 (&pv)[PER]) {
        const int t0 = c0 + t * KT + PER * my_keys;  // this thread's first key of the tile
        const uint4 *ks[PER], *vs[PER];
        if constexpr (APPEND && phase) {
          // cache rows (first tile only), the copied tail block's old
          // slots, then the step's new rows: selects, no branches
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            const int tok = min(t0 + j, c1 - 1);
            const uint64_t rr = static_cast<uint32_t>(max(tok - p0, 0));
            const uint32_t off = (tok & (B - 1)) * DV;
            const uint64_t row = static_cast<uint64_t>(static_cast<uint32_t>(
                                     sm_bt[(tok >> log2_block) - b0])) * blk_units;
            const bool fresh = tok >= p0, copied = tok >= special;
            const uint4 *kf = key_new + rr * key_str, *vf = value_new + rr * value_str;
            const uint4 *kw = key_cow + off, *vw = value_cow + off;
            const uint4 *kr = kc_my + row + off, *vr = vc_my + row + off;
            ks[j] = __builtin_unpredictable(fresh) ? kf : __builtin_unpredictable(copied) ? kw : kr;
            vs[j] = __builtin_unpredictable(fresh) ? vf : __builtin_unpredictable(copied) ? vw : vr;
          }
        } else if constexpr (BIG_B) {
          // the four keys share one block: blocks hold a multiple of 4 keys
          // and t0 is a multiple of 4.  Past the chunk's end the K rows are
          // the block's next slots (scores of keys past the end are masked)
          // and the V rows repeat the chunk's last key (a slot past the
          // sequence may hold anything, and its probability 0 must not meet
          // a NaN); a thread whose keys all lie past the end moves the
          // chunk's last four
          const int tc = min(t0, (c1 - 1) & ~(PER - 1));
          const uint64_t row = static_cast<uint64_t>(static_cast<uint32_t>(
                                   sm_bt[(tc >> log2_block) - b0])) * blk_units;
          const uint32_t slot = (tc & (B - 1)) * DV;
          const uint4* kb = kc_my + row + slot;
          const uint4* vb = vc_my + row + slot;
          // the chunk's last key is at most PER - 1 keys past tc, in its block
          const uint32_t last = static_cast<uint32_t>(c1 - 1 - tc);
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            ks[j] = kb + j * DV;
            vs[j] = vb + min(static_cast<uint32_t>(j), last) * DV;
          }
        } else {
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            const int tok = min(t0 + j, c1 - 1);
            const uint64_t row = static_cast<uint64_t>(static_cast<uint32_t>(
                                     sm_bt[(tok >> log2_block) - b0])) * blk_units;
            const uint32_t off = (tok & (B - 1)) * DV;
            ks[j] = kc_my + row + off;
            vs[j] = vc_my + row + off;
          }
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          pk[j] = load_cached(ks[j]);
          pv[j] = load_cached(vs[j]);
        }
      };
      auto lstore = [&](int buf, int t, const uint4 (&pk)[PER], const uint4 (&pv)[PER]) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          sk[buf][(PER * my_keys + j) * KROW + my_unit] = pk[j];
          sv[buf][(PER * my_keys + j) * VROW + my_unit] = pv[j];
        }
        if constexpr (APPEND && phase) {
          // the row's own tokens, as loaded from the step's rows, to their
          // cache slots (the stores precede the next tile's loads, so the
          // waits for those stay counted)
          const int t0 = c0 + t * KT + PER * my_keys;
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            const int tok = t0 + j;
            if (tok >= L - qlen && tok < c1) {
              const int64_t slot =
                  static_cast<int64_t>(sm_bt[(tok >> log2_block) - b0]) * blk_stride_v +
                  head_off_v + (tok & (B - 1)) * DV + my_unit;
              ap.key_cache[slot] = pk[j];
              ap.value_cache[slot] = pv[j];
            }
          }
        }
      };
      // whether any column of this wave sees a key of the tile (uniform):
      // a tile no column sees leaves every column's softmax as it is
      auto seen = [&](int t) {
        const int t0 = c0 + t * KT;
        return t0 < whi_max && t0 + KT > wlo_min;
      };
      // One tile in two halves: scores and softmax, then the value products.
      // Between them the pipeline stores the next tile and issues the loads
      // of a later one, so that their instructions interleave with the MFMAs.
      auto scores = [&](int t, int buf, uint4 (&phi)[QG][NP]) {
        const int t0 = c0 + t * KT;
        // lane (col, grp) gets the scores of keys 16 st + 4 grp + j of its
        // column in each group; one K fragment feeds both groups
        f32x4 sc[QG][NS];
#pragma unroll
        for (int g = 0; g < QG; ++g)
#pragma unroll
          for (int st = 0; st < NS; ++st) sc[g][st] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // the K fragments of sub-tile st + 1 are read while the MFMAs of
        // sub-tile st run (the scheduler barrier keeps the reads ahead)
        uint4 ka[2][NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) ka[0][k] = sk[buf][col * KROW + k * 4 + grp];
        // a wave issuing MFMAs wins the issue arbitration over one doing its
        // softmax on the same SIMD, so that the two overlap
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          if (st + 1 < NS) {
#pragma unroll
            for (int k = 0; k < NK; ++k)
              ka[(st + 1) & 1][k] = sk[buf][((st + 1) * 16 + col) * KROW + k * 4 + grp];
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int k = 0; k < NK; ++k)
#pragma unroll
            for (int g = 0; g < QG; ++g) sc[g][st] = MM::k32(ka[st & 1][k], qv[g][k], sc[g][st]);
        }
        __builtin_amdgcn_s_setprio(0);
        // a tile inside every column's keys needs no mask (wave-uniform);
        // otherwise key st * 16 + j past this lane's first (t0 + 4 grp) is
        // visible below hi and, with a window, from lw on (a column without
        // a query has hi <= 0 and lw beyond every key)
        const bool masked = !(t0 >= wlo_max && t0 + KT <= min(whi_min, c1));
        if (masked) {
          const int rel = t0 + 4 * grp;
#pragma unroll
          for (int g = 0; g < QG; ++g) {
            const int hi = min(bound[g], c1) - rel;
            const int lw = lo[g] - rel;
            if (window > 0) {
#pragma unroll
              for (int st = 0; st < NS; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const bool vis = (st * 16 + j < hi) & (st * 16 + j >= lw);
                  sc[g][st][j] = vis ? sc[g][st][j] : -INFINITY;
                }
            } else {
#pragma unroll
              for (int st = 0; st < NS; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  sc[g][st][j] = st * 16 + j < hi ? sc[g][st][j] : -INFINITY;
            }
          }
        }
        // Probabilities rounded once to the storage's 16-bit type, two per
        // conversion, for the value products (K = 32 keys per MFMA), and
        // summed as rounded: the output is then exactly a convex combination
        // of the values with these weights, each within 2^-9 (bf16) or
        // 2^-12 (fp16) of its own probability.
        auto probs = [&](int g) {
          float tsum = 0.0f;
#pragma unroll
          for (int sp = 0; sp < NP; ++sp) {
            uint32_t w[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int j = 0; j < 4; j += 2) {
                w[2 * hh + j / 2] = MM::pack2(
                    __builtin_amdgcn_exp2f(fmaf(sc[g][2 * sp + hh][j], scale_log2, -ms[g])),
                    __builtin_amdgcn_exp2f(fmaf(sc[g][2 * sp + hh][j + 1], scale_log2, -ms[g])));
                tsum = MM::sum2(w[2 * hh + j / 2], tsum);
              }
            phi[g][sp] = make_uint4(w[0], w[1], w[2], w[3]);
          }
          return tsum;
        };
        // The reference maximum of a column moves only when the tile's
        // maximum exceeds it by more than 2^8: probabilities stay below 256
        // and the accumulators are rescaled only on such rare jumps.  Once
        // every column of the wave that has a query has a reference, a tile
        // first takes its probabilities against the current references: a
        // lane's sum of at most 256 bounds each of its terms, and only when
        // some lane's sum exceeds that does the wave reduce the maxima
        // across lanes, move the references and take the probabilities
        // again.  Until then every tile reduces the maxima first.
        float tsum[QG];
        bool full = !all_set;
        if (!full) {
          bool over = false;
#pragma unroll
          for (int g = 0; g < QG; ++g) {
            tsum[g] = probs(g);
            over |= tsum[g] > 256.0f;
          }
          full = __any(over);
        }
        if (full) {
          bool set = true;
#pragma unroll
          for (int g = 0; g < QG; ++g) {
            float mt = -INFINITY;
#pragma unroll
            for (int st = 0; st < NS; ++st)
              mt = fmaxf(mt, fmaxf(fmaxf(sc[g][st][0], sc[g][st][1]),
                                   fmaxf(sc[g][st][2], sc[g][st][3])));
            mt = column_max(mt) * scale_log2;
            const float mref = mt > m[g] + 8.0f ? mt : m[g];
            const float mnew = mref == -INFINITY ? 0.0f : mref;
            const float corr = __builtin_amdgcn_exp2f(m[g] - mnew);
            if (__any(mref != m[g])) {
#pragma unroll
              for (int e = 0; e < NE; ++e) o[g][e] *= corr;
            }
            lsum[g] *= corr;
            m[g] = mref;
            ms[g] = mnew;
            set &= (mref != -INFINITY) | !valid[g];
            tsum[g] = probs(g);
          }
          all_set = __all(set);
        }
#pragma unroll
        for (int g = 0; g < QG; ++g) lsum[g] += tsum[g];
      };
      auto values = [&](int buf, const uint4 (&phi)[QG][NP]) {
        const char* vb = reinterpret_cast<const char*>(sv[buf]) + v_read;
        // dim 16 e + col of keys 32 sp + 4 grp + 0..3 and the same + 16 (the
        // order of the probabilities in phi), read VD steps ahead of the
        // MFMAs that take them
        constexpr int VD = 3;
        constexpr int NV = NP * NE;
        uint4 va[VD + 1];
        auto vread = [&](int i) {
          const int sp = i / NE, e = i % NE;
          const uint2 x0 = read_columns(vb + 32 * e + 32 * sp * VROW * 16);
          const uint2 x1 = read_columns(vb + 32 * e + (32 * sp + 16) * VROW * 16);
          return make_uint4(x0.x, x0.y, x1.x, x1.y);
        };
#pragma unroll
        for (int i = 0; i < VD; ++i) va[i] = vread(i);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          if (i + VD < NV) va[(i + VD) % (VD + 1)] = vread(i + VD);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int g = 0; g < QG; ++g)
            o[g][i % NE] = MM::k32(va[i % (VD + 1)], phi[g][i / NE], o[g][i % NE]);
        }
        __builtin_amdgcn_s_setprio(0);
      };
      // LDS holds tile t and t + 1 alternately; registers carry the loads
      // of the tile after, so one tile's rows are in flight while one is
      // computed (pairs of tiles with no exit between them: the waits for
      // the loads in flight stay counted, not full drains)
      uint4 ak[PER], av[PER];
      gload(0, ak, av);
      lstore(0, 0, ak, av);
      gload(1, ak, av);
      __syncthreads();
      uint4 phi[QG][NP];
      int t = 0;
      for (; t + 1 < ntiles; t += 2) {
        const bool s0 = seen(t), s1 = seen(t + 1);
        if (s0) scores(t, 0, phi);
        lstore(1, t + 1, ak, av);
        gload(t + 2, ak, av);
        if (s0) values(0, phi);
        __syncthreads();
        if (s1) scores(t + 1, 1, phi);
        lstore(0, t + 2, ak, av);
        gload(t + 3, ak, av);
        if (s1) values(1, phi);
        __syncthreads();
      }
      if (t < ntiles && seen(t)) {  // an odd last tile, in buffer 0
        scores(t, 0, phi);
        values(0, phi);
      }
    }
  };
  if constexpr (SPLIT) {
    // the partition's keys (a multiple of 16 from its start, so a thread's
    // four keys still share one block)
    range(std::false_type{}, max(lo_min, part * partition_size),
          min(L, (part + 1) * partition_size));
  } else {
    range(std::false_type{}, lo_min, split);
    if constexpr (APPEND) range(std::true_type{}, split, L);
  }

  if (APPEND && ap.slot_mapping && kvh == 0) {
    // the slots of this row's tokens to the mapping
    for (int i = tid; i < qlen; i += NT) {
      const int tok = L - qlen + i;
      ap.slot_mapping[q0 + i] = static_cast<int64_t>(bt_row[tok >> log2_block]) * B + (tok & (B - 1));
    }
  }

#pragma unroll
  for (int g = 0; g < QG; ++g) {
    // per-column sum over the four lane groups (disjoint key slots)
    float l = lsum[g];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!valid[g]) continue;
    if constexpr (SPLIT) {
      // the partial of the column's vector: its reference (natural-log
      // units), its sum and its normalised output, or (-inf, 0, 0) when
      // the partition holds no key it sees; lane (col, grp) holds dims
      // 16 e + 4 grp + j
      const int64_t slot =
          (static_cast<int64_t>(q0 + qi[g]) * num_heads + hq[g]) * num_partitions + part;
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      float* dsto = ws_out + slot * D + 4 * grp;
#pragma unroll
      for (int e = 0; e < NE; ++e) *reinterpret_cast<f32x4*>(dsto + 16 * e) = o[g][e] * inv;
      if (grp == 0) {
        ws_max[slot] = l > 0.0f ? ms[g] * kLn2 : -INFINITY;
        ws_sum[slot] = l;
      }
      continue;
    }
    // lane (col, grp) holds dims 16 e + 4 grp + j of its column: four
    // contiguous dims per e, stored as one 8-byte piece
    uint16_t* dst = static_cast<uint16_t*>(out) +
                    (static_cast<int64_t>(q0 + qi[g]) * num_heads + hq[g]) * D + 4 * grp;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      *reinterpret_cast<uint2*>(dst + 16 * e) =
          make_uint2(MM::pack2(o[g][e][0] * inv, o[g][e][1] * inv),
                     MM::pack2(o[g][e][2] * inv, o[g][e][3] * inv));
  }
}

}  // namespace

int prefill_block_tokens(int group) { return kPrefillWaves * kPrefillGroups * 16 / group; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  int log2_block = 0;
  while ((1 << log2_block) < a.block_size) ++log2_block;
  int log2_group = 0;
  while ((1 << log2_group) < a.num_heads / a.num_kv_heads) ++log2_group;
  const bool split = a.partition_size > 0;
  const dim3 grid(static_cast<uint32_t>((split ? a.num_items : static_cast<int64_t>(a.num_rows)) *
                                        a.num_kv_heads));
  const float sl2 = a.scale * kLog2e;
  // (keys a thread moves per tile: tile x 16 units / threads)
  const bool big = (1 << log2_block) >= kPrefillTile * 16 / (kPrefillWaves * 64);
  const bool append = a.append.qsl != nullptr;
#define PA_PREFILL(DT, BIG, APP, SPL)                                                          \
  hipLaunchKernelGGL((prefill_kernel<DT, BIG, APP, SPL>), grid, dim3(kPrefillWaves * 64), 0,    \
                     stream, a.out, a.query, a.key_cache, a.value_cache, a.block_tables,        \
                     a.bt_stride, a.row_seq, a.row_lens, a.row_qsl, a.work_items, a.num_rows,   \
                     a.num_heads, a.num_kv_heads, log2_block, log2_group, sl2, a.window,        \
                     a.append, a.partition_size, a.num_partitions, a.ws_max, a.ws_sum, a.ws_out)
#define PA_PREFILL_DT(DT)                                  \
  if (split && big) PA_PREFILL(DT, true, false, true);     \
  else if (split) PA_PREFILL(DT, false, false, true);      \
  else if (big && append) PA_PREFILL(DT, true, true, false); \
  else if (big) PA_PREFILL(DT, true, false, false);        \
  else if (append) PA_PREFILL(DT, false, true, false);     \
  else PA_PREFILL(DT, false, false, false)
  if (split && append) return hipErrorInvalidValue;
  if (a.dtype == PA_BF16) {
    PA_PREFILL_DT(PA_BF16);
  } else {
    PA_PREFILL_DT(PA_F16);
  }
#undef PA_PREFILL_DT
#undef PA_PREFILL
  return hipGetLastError();
}

}  // namespace pa
