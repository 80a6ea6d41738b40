// Device helpers shared by the paged decode kernels: storage-dtype traits
// (16-byte vector loads, dot products, conversions, rounding stores) and
// cross-lane sums.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedkv.h"

namespace pa {
namespace dev {

// Tuning constants (overridable at build time with -D):
//   PA_PREFETCH            tiles each wave keeps in flight ahead of the one it consumes
//   PA_VALU_WAVES          waves per workgroup of the vector kernel
//   PA_VALU_WAVES_SHARED   the same when the launch has shared prefix blocks
//                          (fewer, more numerous workgroups keep the sharers of a
//                          block in flight together, so they hit in the caches)
//   PA_MFMA_WAVES          waves per workgroup of the matrix-core kernel
#ifndef PA_PREFETCH
#define PA_PREFETCH 1
#endif
#ifndef PA_VALU_WAVES
#define PA_VALU_WAVES 8
#endif
#ifndef PA_VALU_WAVES_SHARED
#define PA_VALU_WAVES_SHARED 4
#endif
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
#ifndef PA_STREAM_LOADS
#define PA_STREAM_LOADS 1
#endif
constexpr int kPrefetch = PA_PREFETCH;

// 16-byte K/V loads.  Rows read once per launch go through load_stream, which
// marks them non-temporal so they do not displace reusable lines from L2 and
// the Infinity Cache; rows of blocks shared by several sequences (read by
// several workgroups) use load_cached.  PA_STREAM_LOADS=0 makes both plain.
__device__ __forceinline__ uint4 load_cached(const uint4* p) { return *p; }

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
#if PA_STREAM_LOADS
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

// Load kind of a run of tiles, as a type so that each kind gets its own loop.
template <bool NT>
struct LoadKind {
  static constexpr bool streaming = NT;
};
template <bool NT>
__device__ __forceinline__ uint4 load_kv(const uint4* p) {
  if constexpr (NT) return load_stream(p);
  else return load_cached(p);
}

// First tile >= lo that wave `wave` of `nw` owns when tiles are dealt
// round-robin (tile i belongs to wave i mod nw), and how many of its tiles lie
// below hi.
__device__ __forceinline__ void wave_tiles(int lo, int hi, int wave, int nw, int& first,
                                           int& count) {
  first = lo + ((wave - lo) % nw + nw) % nw;
  count = first < hi ? (hi - first + nw - 1) / nw : 0;
}

constexpr int kTile = 16;          // tokens per tile
constexpr int kChunkTokens = 2048;  // tokens whose table entries are staged at once
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- storage traits -------------------------------------------------------
template <int DT>
struct St;

template <>
struct St<PA_F32> {
  static constexpr int VEC = 4;
  using QReg = float4;
  __device__ static QReg load_q(const void* p, int64_t idx) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
  }
  __device__ static QReg zero_q() { return make_float4(0.0f, 0.0f, 0.0f, 0.0f); }
  __device__ static float dot(const QReg& q, const uint4& k) {
    float s = q.x * __uint_as_float(k.x);
    s = fmaf(q.y, __uint_as_float(k.y), s);
    s = fmaf(q.z, __uint_as_float(k.z), s);
    s = fmaf(q.w, __uint_as_float(k.w), s);
    return s;
  }
  __device__ static void to_float(const uint4& v, float (&f)[VEC]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static void store(void* p, int64_t idx, float x) {
    static_cast<float*>(p)[idx] = x;
  }
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

template <>
struct St<PA_F16> {
  static constexpr int VEC = 8;
  using QReg = uint4;  // 8 halves, packed
  __device__ static QReg load_q(const void* p, int64_t idx) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + idx);
  }
  __device__ static QReg zero_q() { return make_uint4(0, 0, 0, 0); }
  __device__ static float d2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  c, false);
  }
  __device__ static float dot(const QReg& q, const uint4& k) {
    float s = d2(q.x, k.x, 0.0f);
    s = d2(q.y, k.y, s);
    s = d2(q.z, k.z, s);
    s = d2(q.w, k.w, s);
    return s;
  }
  __device__ static void to_float(const uint4& v, float (&f)[VEC]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t h = __builtin_bit_cast(half2_t, w[i]);
      f[2 * i] = static_cast<float>(h.x);
      f[2 * i + 1] = static_cast<float>(h.y);
    }
  }
  __device__ static void store(void* p, int64_t idx, float x) {
    static_cast<_Float16*>(p)[idx] = static_cast<_Float16>(x);
  }
};

template <>
struct St<PA_BF16> {
  static constexpr int VEC = 8;
  using QReg = uint4;
  __device__ static QReg load_q(const void* p, int64_t idx) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + idx);
  }
  __device__ static QReg zero_q() { return make_uint4(0, 0, 0, 0); }
  __device__ static float d2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), c, false);
  }
  __device__ static float dot(const QReg& q, const uint4& k) {
    float s = d2(q.x, k.x, 0.0f);
    s = d2(q.y, k.y, s);
    s = d2(q.z, k.z, s);
    s = d2(q.w, k.w, s);
    return s;
  }
  __device__ static void to_float(const uint4& v, float (&f)[VEC]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(void* p, int64_t idx, float x) {
    // round to nearest even; NaN stays a quiet NaN
    uint32_t u = __float_as_uint(x);
    uint16_t b;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      b = static_cast<uint16_t>((u >> 16) | 0x40);
    } else {
      u += 0x7fffu + ((u >> 16) & 1u);
      b = static_cast<uint16_t>(u >> 16);
    }
    static_cast<uint16_t*>(p)[idx] = b;
  }
};

// ---- cross-lane sums -------------------------------------------------------
// Sum over aligned groups of N lanes (N = 8, 16, 32); every lane of a group
// ends with the group sum.  Within a 16-lane DPP row: xor 1, xor 2 (quad
// permutes), then half-row mirror and row mirror; 32 adds a swap of rows.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += __builtin_amdgcn_update_dpp(0.0f, x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  x += __builtin_amdgcn_update_dpp(0.0f, x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  x += __builtin_amdgcn_update_dpp(0.0f, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  if constexpr (N >= 16) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x140, 0xF, 0xF, false);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}


// ---- work units -------------------------------------------------------------
// (sequence, KV head, partition) of this workgroup.  With a work list,
// workgroup b serves item b / H_kv, KV head b % H_kv (items are (sequence,
// partition) pairs, largest first); without one, workgroup b serves
// partition b % grid_parts, KV head (b / grid_parts) % H_kv and sequence
// b / (grid_parts * H_kv), all on grid.x (no 65535 limit of grid.y / z).
struct WorkUnit {
  int s, kvh, p;
};

__device__ __forceinline__ WorkUnit work_unit(const int2* items, int num_kv_heads,
                                              int grid_parts) {
  const uint32_t b = blockIdx.x;
  if (items) {
    const int2 it = items[b / num_kv_heads];
    return {it.x, static_cast<int>(b % num_kv_heads), it.y};
  }
  const uint32_t sh = b / grid_parts;
  return {static_cast<int>(sh / num_kv_heads), static_cast<int>(sh % num_kv_heads),
          static_cast<int>(b % grid_parts)};
}

// ---- the step's cache writes, fused into the attention launch ---------------
// A decode step appends n_s new tokens to every sequence s: positions
// [L_s - n_s, L_s), where L_s = context_lens[s] counts them; their K/V rows are
// rows qsl[s] .. qsl[s+1]-1 of key/value.  If cow_src[s] >= 0 the block that
// holds position L_s - n_s is a fresh copy-on-write copy of block cow_src[s]
// for the slots before the first new token.  Each attention work item
// (s, kv head, token range) writes exactly the rows it is about to read, so
// no other workgroup reads them during the launch.
struct AppendArgs {
  const int32_t* qsl;      // [S + 1] token offsets; nullptr = nothing to write
  const int64_t* cow_src;  // [S] source block or -1; nullptr = no copies
  const uint4* key;        // new rows, 16-byte units
  const uint4* value;
  int64_t key_stride_v;    // units between consecutive tokens
  int64_t value_stride_v;
  uint4* key_cache;        // the caches, writable
  uint4* value_cache;
  int64_t* slot_mapping;   // [T] slots of the new tokens (written), or nullptr
};

template <int LPT, int NT>
__device__ void apply_appends(const AppendArgs& ap, int s, int kvh, int L, int t_begin,
                              int t_end, const int32_t* bt_row, int log2_block,
                              int64_t blk_stride_v, int64_t head_off_v) {
  const int i0 = ap.qsl[s];
  const int n = ap.qsl[s + 1] - i0;
  const int p0 = L - n;  // first new position
  const int B = 1 << log2_block;
  if (n > 0 && ap.cow_src) {
    const int64_t src = ap.cow_src[s];
    const int jb = p0 >> log2_block;
    const int bstart = jb << log2_block;
    if (src >= 0 && bstart >= t_begin && bstart < t_end) {
      const int64_t from = src * blk_stride_v + head_off_v;
      const int64_t to = static_cast<int64_t>(bt_row[jb]) * blk_stride_v + head_off_v;
      const int units = (p0 - bstart) * LPT;  // old slots of the copied block
      for (int u = threadIdx.x; u < units; u += NT) {
        ap.key_cache[to + u] = ap.key_cache[from + u];
        ap.value_cache[to + u] = ap.value_cache[from + u];
      }
    }
  }
  const int a = max(p0, t_begin), b = min(L, t_end);
  const int units = (b > a ? b - a : 0) * LPT;
  for (int u = threadIdx.x; u < units; u += NT) {
    const int t = a + u / LPT, e = u % LPT;
    const int64_t i = i0 + (t - p0);
    const int64_t phys = bt_row[t >> log2_block];
    const int off = t & (B - 1);
    const int64_t dst = phys * blk_stride_v + head_off_v + static_cast<int64_t>(off) * LPT + e;
    ap.key_cache[dst] = ap.key[i * ap.key_stride_v + kvh * LPT + e];
    ap.value_cache[dst] = ap.value[i * ap.value_stride_v + kvh * LPT + e];
    if (kvh == 0 && e == 0 && ap.slot_mapping) ap.slot_mapping[i] = phys * B + off;
  }
  // the caller passes a barrier before any wave reads these rows
}

// ---- matrix-core helpers (16-bit storage only) ---------------------------
// Lane layouts (wave64, probed on gfx950):
//   16x16x32: lane l holds A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16]
//   16x16x16: lane l holds A[l%16][4*(l/16) .. +4] and B[4*(l/16) .. +4][l%16]
//   result:   lane l holds C[4*(l/16) .. +4][l%16]
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <int DT>
struct Mma;

template <>
struct Mma<PA_BF16> {
  __device__ static f32x4 k32(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static f32x4 k16(const uint2& a, const uint2& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  // 16-bit pattern of x rounded to nearest even, and its value as float
  __device__ static uint32_t round16(float x, float& back) {
    const __bf16 h = static_cast<__bf16>(x);
    back = static_cast<float>(h);
    return __builtin_bit_cast(uint16_t, h);
  }
  // a and b rounded to nearest even, a in the low half (one conversion)
  __device__ static uint32_t pack2(float a, float b) {
    const float2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf162_t));
  }
  // acc + the two 16-bit values of p, in fp32 (one dot product with (1, 1))
  __device__ static float sum2(uint32_t p, float acc) {
    const bf162_t one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, p), one, acc, false);
  }
};

template <>
struct Mma<PA_F16> {
  __device__ static f32x4 k32(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static f32x4 k16(const uint2& a, const uint2& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t round16(float x, float& back) {
    const _Float16 h = static_cast<_Float16>(x);
    back = static_cast<float>(h);
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static uint32_t pack2(float a, float b) {
    const float2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
  }
  __device__ static float sum2(uint32_t p, float acc) {
    const half2_t one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, p), one, acc, false);
  }
};

__device__ __forceinline__ uint32_t dword(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// One 16-token tile of one wave: scores S^T = K Q^T on the matrix cores, the
// online softmax of every head column (vis[j]: whether this lane's column
// sees token grp + 4j of the tile), and O^T += V^T P^T with P split into a
// 16-bit head and remainder.  (m, lsum) are the column's running maximum
// (log2 domain) and the lane's partial sum; o its accumulator chunks.
template <int DT>
__device__ __forceinline__ void mfma_tile_update(const uint4 (&kr)[4], const uint4 (&vr)[4],
                                                 const uint4 (&qv)[4], const bool (&vis)[4],
                                                 float scale_log2, float& m, float& lsum,
                                                 f32x4 (&o)[8]) {
  using MM = Mma<DT>;
  f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) sc = MM::k32(kr[k], qv[k], sc);
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = vis[j] ? sc[j] * scale_log2 : -INFINITY;
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
    for (int e = 0; e < 8; ++e) o[e] *= corr;
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
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    const int w = e >> 1;
    uint2 a;
    a.x = __builtin_amdgcn_perm(dword(vr[1], w), dword(vr[0], w), sel);
    a.y = __builtin_amdgcn_perm(dword(vr[3], w), dword(vr[2], w), sel);
    o[e] = MM::k16(a, phi, o[e]);
    o[e] = MM::k16(a, plo, o[e]);
  }
}

}  // namespace dev
}  // namespace pa
