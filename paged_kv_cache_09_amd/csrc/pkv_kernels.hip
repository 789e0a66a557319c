// HIP kernels for paged KV-cache decode on MI355X (gfx950, wave64).
//
//  decode_kernel  — per wavefront: a run of (kv head, sequence, block) tiles;
//                   gathers 16 x head_dim K and V tiles through the block table
//                   with wide per-lane loads, computes q.K^T for all query
//                   heads of the GQA group sharing the kv head, keeps an fp32
//                   online softmax and accumulates P.V. A run that covers a
//                   whole (kv head, sequence) writes the normalised output;
//                   otherwise it leaves an unnormalised partial (max, sum, o)
//                   in HBM (split form) or in LDS for another wave of its
//                   eight-wave workgroup (bins form). In the split form the
//                   first workgroups can be shared-prefix items: a prompt
//                   several sequences share through their tables, read once
//                   per group of them.
//  reduce_kernel  — merges the partials of one (sequence, q head):
//                   out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i.
//                   (A merge by the last-finishing wavefront would save this
//                   launch, but publishing partials across XCDs needs an
//                   agent-scope release, an L2 write-back on this chip, which
//                   measured ~3x slower than the extra launch.)
//  append_kernel  — scatters each sequence's new K/V rows into the pool at its slot.
//  append_q8_kernel / append_q4_kernel — the same for a q8_0 / q4_0 cache:
//                   quantise each 32-value group of the bf16 new rows to int8
//                   or 4-bit codes and an fp16 scale.
//  upload_kernel  — copies a packed metadata image from pinned host memory to
//                   the device on the launch stream (no copy-engine hand-off).
//  copy_blocks_kernel — copy-on-write: whole K/V blocks src -> dst for every layer.
//
// What is computed follows the pages: the cache is split into 16-token blocks
// reached through a block table (ahmedhaies.com, "PagedAttention: why LLM
// serving wastes most GPU memory", "The solution: borrow virtual memory from
// the OS"), decode reads the whole cache and appends one key/value per step
// (news.hamidun.com "KV-Cache", prefill/decode paragraph), and grouped-query
// heads share one stored K/V head (ssdnodes.com, "KV cache vs prompt cache",
// GQA paragraph). Decode is bound by memory bandwidth (ssdnodes.com, same
// page, "What the KV cache holds"), so every tile is read exactly once, with
// 16-byte lanes (for q8_0 and q4_0 the tile layout puts each lane's codes in
// one run);
// q.K^T of the GQA group runs on 16x16 MFMA tiles, the softmax on the fp32
// VALU, and P.V on the fp32 VALU or, where it bounds the loop (q4_0, q8_0) or
// serves 16 rows (shared-prefix items), on MFMA with the weights in 16-bit
// parts (quantised codes as exact fp16 subnormals).
#include "pkv_internal.h"

#include <mutex>

namespace pkv {
namespace {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_Q8 = 3, DT_Q4 = 4 };
// Context lengths handed to the decode kernel carry a flag in bit 30.
constexpr int kLenMask = (1 << 30) - 1;

#ifdef PKV_TIMELINE
// Diagnostic build only: per wave (start, first tile done, loop end, merge
// end, xcc | tiles << 8 | segments << 24, wave id, after the barrier, 0) in
// s_memrealtime ticks.
__device__ long long pkv_tl[8 * 8192];
#endif

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// q8_0 tile layout: the codes of a block (block_size rows of D int8 codes) are
// stored in the order the decode's lanes read them, so that every 16-byte
// load instruction of a wave reads 1 KiB (R = min(block size, 16) rows)
// contiguously. Rows are taken R at a time (u = r / R, rr = r % R); with
// P = D / 8 chunks of 8 codes per row and NV = P / 4:
//   K: chunk w = 4k + q (group k, quarter q) of row r at
//      u*R*D + (k/2)*R*64 + (q*R + rr)*16 + (k%2)*8
//      (lane (token rr, quarter q) reads its groups 2c, 2c+1 as 16 bytes at
//      c*R*64 + lane*16);
//   V: chunk w of row r at u*R*D + ((rr%NV)/2)*R*64 + ((rr/NV)*P + w)*16 +
//      (rr%2)*8 (lane (chunk w, rows NV*v .. NV*v+NV-1) reads two rows' chunks
//      as 16 bytes at c*R*64 + lane*16).
// Scales follow the codes as before: K [row][group], V [group][row].
template <int D>
__device__ __forceinline__ int q8_chunk_offset(bool is_v, int r, int w, int bs) {
  constexpr int P = D / 8, NV = P / 4;
  const int R = bs < 16 ? bs : 16, u = r / R, rr = r % R;
  if (is_v) return u * R * D + ((rr % NV) >> 1) * R * 64 + ((rr / NV) * P + w) * 16 + (rr & 1) * 8;
  const int k = w >> 2, q = w & 3;
  return u * R * D + (k >> 1) * R * 64 + (q * R + rr) * 16 + (k & 1) * 8;
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Bytes of one stored element (q8_0: one int8 code; q4_0: counted as one
// here, the tile layout packs two codes per byte; scales are extra).
template <int DT>
struct Elem {
  static constexpr int bytes = DT == DT_F32 ? 4 : (DT == DT_Q8 || DT == DT_Q4) ? 1 : 2;
};

__device__ __forceinline__ u32x4 ld16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const char* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ unsigned ld4(const char* p) {
  return *reinterpret_cast<const unsigned*>(p);
}
// A load of a wave-uniform int that stays on the vector memory path: a scalar
// load would be counted by lgkmcnt, which the tile loop's LDS exchanges also
// wait on, so a prefetch in flight would stall them. The zero offset is opaque
// to the compiler (a per-lane register), which keeps the load a vector load.
__device__ __forceinline__ int vld(const int32_t* p) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return p[z];
}
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
// Pool tiles are read once per launch: nontemporal loads (the nt cache
// policy) stream them past the caches.
__device__ __forceinline__ u32x4 nt16(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 nt8(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ unsigned nt4(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p));
}
#ifndef PKV_NT_SCALES
#define PKV_NT_SCALES 0
#endif
__device__ __forceinline__ u32x2 ldsc8(const char* p) { return PKV_NT_SCALES ? nt8(p) : ld8(p); }
__device__ __forceinline__ unsigned ldsc4(const char* p) { return PKV_NT_SCALES ? nt4(p) : ld4(p); }

// fp16 halves of a 32-bit word, as fp32.
__device__ __forceinline__ float half_lo(unsigned u) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu));
}
__device__ __forceinline__ float half_hi(unsigned u) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16));
}
__device__ __forceinline__ unsigned half_bits(float f) {
  return (unsigned)__builtin_bit_cast(unsigned short, (_Float16)f);
}

// Byte b of w as a signed 8-bit integer, in fp32.
__device__ __forceinline__ float sbyte(unsigned w, int b) {
  return (float)(int)(signed char)(w >> (8 * b));
}

// The upper halves of two fp32 values as one bf16 pair (exact for the small
// integers this is used on: their fp32 encodings end in 16 zero bits).
__device__ __forceinline__ unsigned bf16_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(unsigned, hi), __builtin_bit_cast(unsigned, lo),
                               0x07060302u);
}

// 8 int8 codes -> 8 bf16 values (exact), an MFMA operand.
__device__ __forceinline__ u32x4 codes_to_bf16(u32x2 c) {
  const unsigned w0 = c[0], w1 = c[1];
  u32x4 r;
  r[0] = bf16_pair(sbyte(w0, 0), sbyte(w0, 1));
  r[1] = bf16_pair(sbyte(w0, 2), sbyte(w0, 3));
  r[2] = bf16_pair(sbyte(w1, 0), sbyte(w1, 1));
  r[3] = bf16_pair(sbyte(w1, 2), sbyte(w1, 3));
  return r;
}

// 8 int8 codes -> the 8 values (128 + code) x 2^-24 as fp16, in natural order,
// an MFMA operand: 128 + code is the code's byte with its top bit flipped, and
// as fp16 bits over a zero high byte it is that many units of the smallest
// subnormal, exactly (the MFMA keeps subnormal inputs). The 128 is taken off
// through the MFMA's accumulator input.
__device__ __forceinline__ u32x4 codes_to_f16_128(u32x2 c) {
  const unsigned w0 = c[0] ^ 0x80808080u, w1 = c[1] ^ 0x80808080u;
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(0u, w0, 0x0c010c00u);  // (w0.b0, 0, w0.b1, 0)
  r[1] = __builtin_amdgcn_perm(0u, w0, 0x0c030c02u);
  r[2] = __builtin_amdgcn_perm(0u, w1, 0x0c010c00u);
  r[3] = __builtin_amdgcn_perm(0u, w1, 0x0c030c02u);
  return r;
}

// 8 packed 4-bit codes (code j in bits 4j .. 4j+3) -> an fp16 MFMA operand
// of subnormals, in the slot order 0 4 1 5 2 6 3 7: codes 0, 4, 2, 6 as c x
// 2^-24 and codes 1, 5, 3, 7 as 16c x 2^-24 (exact: fp16 bits below 0x400
// count units of the smallest subnormal, and the MFMA keeps them), each
// dword one mask of the word or of the word shifted by 8. The q operand is
// put in the same order, its odd elements divided by 16.
__device__ __forceinline__ u32x4 nibbles_to_f16(unsigned w) {
  const unsigned w8 = w >> 8;
  return u32x4{w & 0x000f000fu, w & 0x00f000f0u, w8 & 0x000f000fu, w8 & 0x00f000f0u};
}

// Code values in fp32: 8 int8 codes (q8_0), or 8 packed 4-bit codes 0..15
// (q4_0: the caller takes off 8 times the weight sum).
__device__ __forceinline__ void code_vals(u32x2 c, float (&v)[8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[b] = sbyte(c[0], b);
    v[4 + b] = sbyte(c[1], b);
  }
}
__device__ __forceinline__ void code_vals(unsigned w, float (&v)[8]) {
  unsigned lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
  // hide the masks from the optimiser: it would otherwise extract every
  // nibble with its own bit-field op instead of converting bytes directly
  asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[2 * b] = (float)((lo >> (8 * b)) & 0xffu);
    v[2 * b + 1] = (float)((hi >> (8 * b)) & 0xffu);
  }
}

// q8_0 quantisation of 8 values of one 32-value group whose max |x| is amax:
// scale d = amax / 127 (fp32, stored as fp16), codes round(x * (1 / d)),
// halves away from zero (llama.cpp's Q8_0 format, the q8_0 cache type of
// ssdnodes.com, "KV cache vs prompt cache", "Four ways to make the KV cache
// smaller"). Returns the 8 codes; *d_out gets the fp32 scale.
__device__ __forceinline__ u32x2 q8_codes(const float (&x)[8], float amax, float* d_out) {
  const float d = amax / 127.f;
  const float id = d != 0.f ? 1.f / d : 0.f;
  unsigned w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = (int)__builtin_roundf(x[j] * id);
    w[j >> 2] |= ((unsigned)c & 0xffu) << (8 * (j & 3));
  }
  *d_out = d;
  return u32x2{w[0], w[1]};
}

// q4_0 (llama.cpp's Q4_0 format, the q4_0 cache type of ssdnodes.com, "KV
// cache vs prompt cache", "Four ways to make the KV cache smaller"): a group's
// scale is d = m / -8, m its value of largest magnitude (the first on ties,
// +0 for an all-zero group); codes q = min(15, trunc(x * (1 / d) + 8.5)) with
// the product and the sum rounded separately; value (q - 8) * d.
//
// Largest-magnitude value among this lane's 8 values of a group (element
// indices base .. base+7 inside the group): (|m|, m, index), (0, +0, 32) if
// all are zero.
__device__ __forceinline__ void q4_pick(const float (&x)[8], int base, float& a, float& m,
                                        int& idx) {
  a = 0.f;
  m = 0.f;
  idx = 32;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float ax = __builtin_fabsf(x[j]);
    if (ax > a) {
      a = ax;
      m = x[j];
      idx = base + j;
    }
  }
}
// Combine with the lane `off` away (both lanes end with the same pick).
__device__ __forceinline__ void q4_pick_xor(float& a, float& m, int& idx, int off) {
  const float a2 = __shfl_xor(a, off, 64), m2 = __shfl_xor(m, off, 64);
  const int i2 = __shfl_xor(idx, off, 64);
  if (a2 > a || (a2 == a && i2 < idx)) {
    a = a2;
    m = m2;
    idx = i2;
  }
}
// fp16 bits of the scale d = m / -8: -0 for an all-zero group (m = +0). The
// zero case is spelled out: the compiler may fuse the fp16 conversion with
// the product into one fma whose +0 addend turns -0 into +0.
__device__ __forceinline__ unsigned q4_scale_bits(float m, float d) {
  return m == 0.f ? 0x8000u : half_bits(d);
}
// The 8 codes (code j in bits 4j .. 4j+3) of 8 values under the fp32 scale d.
__device__ __forceinline__ unsigned q4_codes(const float (&x)[8], float d) {
#pragma clang fp contract(off)
  const float id = d != 0.f ? 1.f / d : 0.f;
  unsigned w = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float t = x[j] * id;
    t = t + 8.5f;
    w |= (unsigned)min(15, (int)t) << (4 * j);
  }
  return w;
}

// Bit casts from one 32-bit lane of a u32x4. The element is copied to a
// scalar first: __builtin_bit_cast applied directly to a vector element
// expression reads element 0 whatever the index.
template <typename T>
__device__ __forceinline__ T lane_as(u32x4 v, int i) {
  const unsigned u = v[i];
  return __builtin_bit_cast(T, u);
}

// 16 bytes of cache elements -> fp32 values.
template <int DT>
__device__ __forceinline__ void to_f32(u32x4 w, float* out) {
  if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned u = w[i];
      out[2 * i] = __builtin_bit_cast(float, u << 16);
      out[2 * i + 1] = __builtin_bit_cast(float, u & 0xffff0000u);
    }
  } else if constexpr (DT == DT_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = lane_as<f16x2>(w, i);
      out[2 * i] = (float)h[0];
      out[2 * i + 1] = (float)h[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = lane_as<float>(w, i);
  }
}

__device__ __forceinline__ float xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Merge the n partial results (m_i, l_i, o_i) of one (kv head, sequence)
// segment for query head slot hh, stored at partial indices first .. first+n-1:
//   out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
// One wavefront; lane handles head_dim/64 consecutive output elements. Up to
// 64 partials are merged with all loads issued before any arithmetic (lane i
// holds partial i's max and sum, the first eight outputs are prefetched);
// more partials take a strided path.
template <int D, int GP>
__device__ __forceinline__ void merge_partials(const float* part_o, const float* part_ml,
                                               size_t first, int n, int hh, float* dst,
                                               int lane) {
  constexpr int PER = D / 64;
  constexpr int PF = 8;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  float den = 0.f;
  if (n <= 64) {
    float mi = -__builtin_inff(), li = 0.f;
    if (lane < n) {
      mi = part_ml[((first + lane) * GP + hh) * 2];
      li = part_ml[((first + lane) * GP + hh) * 2 + 1];
    }
    float ob[PF][PER];
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
      for (int e = 0; e < PER; ++e)
        ob[u][e] = u < n ? part_o[((first + u) * GP + hh) * D + lane * PER + e] : 0.f;
    float M = mi;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, xor_f(M, off));
    const float wi = lane < n ? __builtin_amdgcn_exp2f(mi - M) : 0.f;
    den = wi * li;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) den += xor_f(den, off);
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const float wu = __shfl(wi, u, 64);
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(wu, ob[u][e], o[e]);
    }
    for (int u = PF; u < n; ++u) {
      const float wu = __shfl(wi, u, 64);
#pragma unroll
      for (int e = 0; e < PER; ++e)
        o[e] = __builtin_fmaf(wu, part_o[((first + u) * GP + hh) * D + lane * PER + e], o[e]);
    }
  } else {
    float M = -__builtin_inff();
    for (int i = lane; i < n; i += 64) M = fmaxf(M, part_ml[((first + i) * GP + hh) * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, xor_f(M, off));
    for (int i = lane; i < n; i += 64) {
      const float* ml = part_ml + ((first + i) * GP + hh) * 2;
      den += __builtin_amdgcn_exp2f(ml[0] - M) * ml[1];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) den += xor_f(den, off);
    int i = 0;
    for (; i + 4 <= n; i += 4) {  // four independent partials in flight
      float wgt[4], src[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wgt[u] = part_ml[((first + i + u) * GP + hh) * 2];
#pragma unroll
        for (int e = 0; e < PER; ++e)
          src[u][e] = part_o[((first + i + u) * GP + hh) * D + lane * PER + e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wu = __builtin_amdgcn_exp2f(wgt[u] - M);
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(wu, src[u][e], o[e]);
      }
    }
    for (; i < n; ++i) {
      const float wu = __builtin_amdgcn_exp2f(part_ml[((first + i) * GP + hh) * 2] - M);
#pragma unroll
      for (int e = 0; e < PER; ++e)
        o[e] = __builtin_fmaf(wu, part_o[((first + i) * GP + hh) * D + lane * PER + e], o[e]);
    }
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[lane * PER + e] = o[e] * inv;
}

// Softmax bookkeeping is in the log2 domain. A running maximum is raised
// (and the accumulators rescaled) only when a score exceeds it by more than
// this many binary orders; weights stay <= 2^kLazy, far from fp32 overflow,
// and the result is the same softmax up to rounding.
constexpr float kLazy = 8.f;

// Row-wide (16-lane DPP row) all-reductions.
template <int CTRL>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, row_ror<0x128>(v));  // row_ror:8
  v = fmaxf(v, row_ror<0x124>(v));  // row_ror:4
  v = fmaxf(v, row_ror<0x122>(v));  // row_ror:2
  return fmaxf(v, row_ror<0x121>(v));  // row_ror:1
}
__device__ __forceinline__ float row_sum(float v) {
  v += row_ror<0x128>(v);
  v += row_ror<0x124>(v);
  v += row_ror<0x122>(v);
  return v + row_ror<0x121>(v);
}

// How compute_tile treats a tile's P.V on the MFMA path: at once (0), left
// pending for the next tile (1), or together with the pending one (2).
template <int M>
struct PvMode {
  static constexpr int value = M;
};

// Orders this wavefront's LDS writes before its later LDS reads by other
// lanes (a wave's LDS operations complete in order; this keeps the compiler
// from moving them). Only this wave takes part.
// true when pred holds in any active lane: the ballot's mask compared in
// scalar registers (no vector instructions, unlike a vote through a lane)
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 1.0 in every fp16 slot of an MFMA operand.
__device__ __forceinline__ f16x8 ones_f16() {
  return __builtin_bit_cast(f16x8, u32x4{0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u});
}

// x ~ hi + lo: hi rounded toward zero to fp16, lo = x - hi (exact in fp32)
// rounded to fp16: ~22 significant bits together.
__device__ __forceinline__ void split_f16(const float (&x)[4], f16x4& hi, f16x4& lo) {
  typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
  const f16x2v h01 = __builtin_bit_cast(f16x2v, __builtin_amdgcn_cvt_pkrtz(x[0], x[1]));
  const f16x2v h23 = __builtin_bit_cast(f16x2v, __builtin_amdgcn_cvt_pkrtz(x[2], x[3]));
  hi = f16x4{h01[0], h01[1], h23[0], h23[1]};
  lo = f16x4{(_Float16)(x[0] - (float)h01[0]), (_Float16)(x[1] - (float)h01[1]),
             (_Float16)(x[2] - (float)h23[0]), (_Float16)(x[3] - (float)h23[1])};
}

// One 16-byte piece of the q.K^T contraction on the matrix cores:
// A = q (16 rows = heads of the group, zero-padded), B = K^T (16 columns =
// the tile's tokens). Lane l supplies row/column l%16 and the same 16 bytes
// of head_dim for both operands, so the products pair up correctly whatever
// order the instruction walks its K dimension in.
// One MFMA 16x16x16 of P.V in a 2-byte type: 4 weights (A) x 4 rows of one
// column (B) per lane.
template <int DT>
__device__ __forceinline__ f32x4 pv_mfma(u32x2 a, u32x2 b, f32x4 acc) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), acc, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 qk_piece(u32x4 q, u32x4 k, f32x4 acc) {
  if constexpr (DT == DT_BF16) {
    const u32x4 qq = q, kk = k;
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qq),
                                                   __builtin_bit_cast(bf16x8, kk), acc, 0, 0, 0);
  } else if constexpr (DT == DT_F16) {
    const u32x4 qq = q, kk = k;
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, qq),
                                                  __builtin_bit_cast(f16x8, kk), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(lane_as<float>(q, i), lane_as<float>(k, i), acc,
                                                 0, 0, 0);
    return acc;
  }
}

// One lane's share of a (block, kv head) K and V tile.
//   fp32 / fp16 / bf16: NP 16-byte K pieces (lane (t16, kg) holds bytes
//   kg*16 + 64*k of row t16) and NV 16-byte V chunks (chunk vc of rows
//   vr + RPI*i).
//   q8_0 / q4_0: NP 8-byte / 4-byte K pieces (codes 32*k + 8*kg .. +8 of row
//   t16, one piece per 32-code scale group) with that row's NP fp16 scales,
//   and NV 8-byte / 4-byte V chunks (codes 8*vc .. +8 of rows NV*vr + i) with
//   those rows' scales of group vc/4.
template <int DT, int D>
struct TileRegs {
  static constexpr int RB = D * Elem<DT>::bytes;
  static constexpr int NP = RB / 64, CPR = RB / 16, RPI = 64 / CPR, NV = 16 / RPI;
  u32x4 k[NP];
  u32x4 v[NV];
};
template <int D>
struct TileRegs<DT_Q8, D> {
  static constexpr int NP = D / 32, CPR = D / 8, RPI = 64 / CPR, NV = 16 / RPI;
  u32x2 k[NP];
  u32x2 v[NV];
  unsigned ks[NP / 2];  // fp16 pairs: scale of group k in half k % 2 of ks[k / 2]
  unsigned vs[NV / 2];  // fp16 pairs: scale of row NV*vr + i in half i % 2 of vs[i / 2]
};
// q4_0: as q8_0 with 4-byte pieces and chunks (8 packed codes each).
template <int D>
struct TileRegs<DT_Q4, D> {
  static constexpr int NP = D / 32, CPR = D / 8, RPI = 64 / CPR, NV = 16 / RPI;
  unsigned k[NP];
  unsigned v[NV];
  unsigned ks[NP / 2];
  unsigned vs[NV / 2];
};

// Shared-prefix work items (split form; run by the first workgroups of the
// decode launch, next to the private runs): a group of up to 16 / GP sequences whose
// tables name the same blocks for their first full tiles (a common prompt,
// shared through the block table as the pages describe) reads those tiles
// once. One wave per (group, kv head, chunk of the shared tiles): the MFMA's
// 16 rows hold member x head (2 x 8 for 8 q heads per kv head, 4 x 4, 8 x 2, 16 x 1)
// in q.K^T and in P.V, so one tile read serves every member. Each (member,
// head) leaves an unnormalised partial (max, sum, output) in the slot just
// before its own private run's partials, where the reduce merges it. 2-byte
// caches, head_dim 128: K pieces and V chunks are loaded as in decode_kernel;
// P.V takes the weights in parts of the cache's 16-bit type (bf16: three, 24
// bits together; fp16: a high and a low part, ~22 bits; the weights are
// <= 2^kLazy).
template <int DT, int GP, int BS>
__device__ __forceinline__ void prefix_item(const DecodeParams& p, int item) {
  static_assert(DT == DT_F16 || DT == DT_BF16, "2-byte caches");
  constexpr int D = 128, RB = 2 * D, NP = 4, NV = 4;  // as TileRegs<DT, 128>
  constexpr int TILE = BS * RB;
  using TR = TileRegs<DT, D>;
  __shared__ float pl_all[2][16 * 16];  // weights [token][row], by parity
  const int lane = threadIdx.x;
  const int* it = p.items + kItemInts * item;
  const int grp = it[0], g = it[1], t0 = it[2], t1 = it[3], chunk = it[4];
  const int* gr = p.groups + kGroupInts * grp;
  const int count = gr[0], leader = gr[1], nchunks = gr[2];
  const int* members = gr + 3;
  const int t16 = lane & 15, kg = lane >> 4;  // q.K: token column, row block
  const int vc = lane & 15, vr = lane >> 4;   // V chunk, row group (rows vr + 4i)

  // q rows: A row r = member r / GP, head r % GP (zero past the group)
  u32x4 qv[NP];
  {
    const int mq = t16 / GP, hq = t16 % GP;
    const bool real = mq < count && hq < p.group;
    const int sq = members[real ? mq : 0];
    const char* qr = reinterpret_cast<const char*>(p.q) +
                     ((size_t)sq * p.q_heads + (size_t)g * p.group + (real ? hq : 0)) * RB +
                     kg * 16;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const u32x4 v = ld16(qr + k * 64);
      qv[k] = real ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // block-table entries of the chunk, one per lane (<= 32 tiles: <= 64 entries)
  const int32_t* bt_row = p.bt + (size_t)leader * p.bt_stride;
  const int e0 = BS == 32 ? (t0 >> 1) : BS == 8 ? 2 * t0 : t0;
  const int ne = BS == 32 ? ((t1 + 1) >> 1) - (t0 >> 1) : BS == 8 ? 2 * (t1 - t0) : t1 - t0;
  const int my_ent = lane < ne ? bt_row[e0 + lane] : 0;
  const char* kbase = reinterpret_cast<const char*>(p.k) + (size_t)g * TILE;
  const char* vbase = reinterpret_cast<const char*>(p.v) + (size_t)g * TILE;
  const size_t blk_stride = (size_t)p.kv_heads * TILE;
  // tile j (absolute): rows r of the tile live in block (a or b), row rib(r)
  auto load = [&](int j, TR& t) {
    int a, b, half;
    if constexpr (BS == 16) {
      a = b = __builtin_amdgcn_readlane(my_ent, j - t0);
      half = 0;
    } else if constexpr (BS == 32) {
      a = b = __builtin_amdgcn_readlane(my_ent, (j >> 1) - (t0 >> 1));
      half = j & 1;
    } else {
      a = __builtin_amdgcn_readlane(my_ent, 2 * (j - t0));
      b = __builtin_amdgcn_readlane(my_ent, 2 * (j - t0) + 1);
      half = 0;
    }
    auto blk = [&](int r) { return BS == 8 && r >= 8 ? b : a; };
    auto rib = [&](int r) { return BS == 8 ? (r & 7) : BS == 32 ? 16 * half + r : r; };
    const char* kt = kbase + (size_t)blk(t16) * blk_stride + rib(t16) * RB + kg * 16;
#pragma unroll
    for (int k = 0; k < NP; ++k) t.k[k] = ld16(kt + k * 64);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int r = vr + 4 * i;
      t.v[i] = ld16(vbase + (size_t)blk(r) * blk_stride + rib(r) * RB + vc * 16);
    }
  };

  float m[4], lsum[4];  // rows 4 * kg + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -__builtin_inff();
    lsum[i] = 0.f;
  }
  f32x4 acc[8];  // output block nt: rows 4 * (lane / 16) + i, column 8 * (lane % 16) + nt
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  int parity = 0;

  auto compute = [&](const TR& t) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NP; ++k) sacc = qk_piece<DT>(qv[k], t.k[k], sacc);
    float s2[4];
    bool over = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s2[i] = sacc[i] * p.scale_log2;  // the shared tiles are full
      over |= s2[i] > m[i] + kLazy;
    }
    if (wave_any(over)) {
      // the rows of lane's scores are the rows of its output blocks
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mn = fmaxf(m[i], row_max(s2[i]));
        const float a = __builtin_amdgcn_exp2f(m[i] - mn);
        lsum[i] *= a;
        m[i] = mn;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[nt][i] *= a;
      }
    }
    float* pl = pl_all[parity];
    parity ^= 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pw = __builtin_amdgcn_exp2f(s2[i] - m[i]);
      lsum[i] += pw;
      pl[t16 * 16 + 4 * kg + i] = pw;
    }
    wave_sync();
    // A: row lane % 16, k = tokens vr + 4 * i (the rows of this lane's V chunks)
    float pa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pa[i] = pl[(vr + 4 * i) * 16 + (lane & 15)];
    u32x2 ahi, alo, alo2;
    if constexpr (DT == DT_BF16) {
      // three truncated bf16 parts, each of what the ones before leave (exact
      // fp32 differences): 24 bits together
      unsigned hb[4], mb[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = __builtin_bit_cast(unsigned, pa[i]) & 0xffff0000u;
        const float r1 = pa[i] - __builtin_bit_cast(float, hb[i]);
        mb[i] = __builtin_bit_cast(unsigned, r1) & 0xffff0000u;
        lb[i] = __builtin_bit_cast(unsigned, r1 - __builtin_bit_cast(float, mb[i]));
      }
      ahi = u32x2{__builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u),
                  __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u)};
      alo = u32x2{__builtin_amdgcn_perm(mb[1], mb[0], 0x07060302u),
                  __builtin_amdgcn_perm(mb[3], mb[2], 0x07060302u)};
      alo2 = u32x2{__builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u),
                   __builtin_amdgcn_perm(lb[3], lb[2], 0x07060302u)};
    } else {
      const f16x2 h01 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(pa[0], pa[1]));
      const f16x2 h23 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(pa[2], pa[3]));
      const f16x2 l01 = {(_Float16)(pa[0] - (float)h01[0]), (_Float16)(pa[1] - (float)h01[1])};
      const f16x2 l23 = {(_Float16)(pa[2] - (float)h23[0]), (_Float16)(pa[3] - (float)h23[1])};
      ahi = u32x2{__builtin_bit_cast(unsigned, h01), __builtin_bit_cast(unsigned, h23)};
      alo = u32x2{__builtin_bit_cast(unsigned, l01), __builtin_bit_cast(unsigned, l23)};
    }
    // B for block nt: column 8 * vc + nt of the 4 rows (element nt of each chunk)
    u32x2 bv[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const unsigned sel = (nt & 1) ? 0x07060302u : 0x05040100u;
      bv[nt] = u32x2{__builtin_amdgcn_perm(t.v[1][nt >> 1], t.v[0][nt >> 1], sel),
                     __builtin_amdgcn_perm(t.v[3][nt >> 1], t.v[2][nt >> 1], sel)};
      acc[nt] = pv_mfma<DT>(ahi, bv[nt], acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = pv_mfma<DT>(alo, bv[nt], acc[nt]);
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt] = pv_mfma<DT>(alo2, bv[nt], acc[nt]);
    }
  };

  TR t[2];
  load(t0, t[0]);
  for (int j = t0; j < t1; j += 2) {
    // request the next tile (the last one again past the end: a cache hit)
    load(min(j + 1, t1 - 1), t[1]);
    __builtin_amdgcn_sched_barrier(0);
    compute(t[0]);
    if (j + 1 < t1) {
      load(min(j + 2, t1 - 1), t[0]);
      __builtin_amdgcn_sched_barrier(0);
      compute(t[1]);
    }
  }

  // partials of the real (member, head) rows
  float lt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lt[i] = row_sum(lsum[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * kg + i, mr = r / GP, hr = r % GP;
    if (mr < count && hr < p.group) {
      const int sm = members[mr];
      const int seg = g * p.batch + sm;
      const size_t idx =
          (size_t)(seg + 1) * p.seg_stride - 1 + p.seg_w0[seg] - nchunks + chunk;
      float* o = p.part_o + (idx * GP + hr) * D + 8 * vc;
      *reinterpret_cast<f32x4*>(o) = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
      *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
      if (t16 == 0) {
        p.part_ml[(idx * GP + hr) * 2 + 0] = m[i];
        p.part_ml[(idx * GP + hr) * 2 + 1] = lt[i];
      }
    }
  }
}

// Two launch forms share this body:
//   BINS = false: one wave per workgroup; a wave covers a contiguous run of
//     the kv-head-major tile space; segments split between waves are merged
//     by reduce_kernel from global partials.
//   BINS = true: eight waves per workgroup, one workgroup per bin: a set of
//     whole (kv head, sequence) segments packed by the host so that bins are
//     equally loaded; the bin's tiles are split evenly between its waves and
//     a segment split between them is merged in LDS at the end (no partials
//     in HBM, no reduce launch).
// BS: tokens per pool block (8, 16 or 32). Work is always counted in 16-token
// tiles: a tile is one block (16), half of one (32), or two blocks (8).
template <int DT, int D, int GP, bool BINS, int BS>
__global__ __launch_bounds__(BINS ? 64 * kBinWaves : 64) void decode_kernel(DecodeParams p) {
  constexpr bool Q8 = DT == DT_Q8, Q4 = DT == DT_Q4, QN = Q8 || Q4;
  using TR = TileRegs<DT, D>;
  constexpr int RB = D * Elem<DT>::bytes;  // bytes per K/V row (unquantised caches)
  constexpr int CB = Q4 ? D / 2 : D;       // code bytes per row (quantised caches)
  constexpr int QB = QN ? 2 * D : RB;      // bytes per q / new K,V row (bf16 when quantised)
  constexpr int NP = TR::NP;               // K pieces per lane per tile (= q pieces)
  constexpr int CPR = TR::CPR;             // V chunks per row
  constexpr int RPI = TR::RPI;             // rows covered by one V load instruction
  constexpr int NV = TR::NV;               // V loads per lane per tile
  constexpr int EPC = QN ? 8 : 16 / Elem<DT>::bytes;  // elements per V chunk
  constexpr int NG = GP >= 4 ? GP / 4 : 1;  // lane groups (of 16) holding real heads
  constexpr int HPG = GP >= 4 ? 4 : GP;     // heads per lane group
  // bytes of one (block, kv head) tile of the pool: BS rows (+ scales when quantised)
  constexpr int TILE = QN ? BS * CB + BS * (D / 32) * 2 : BS * RB;
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  // Tile buffers per wave (tiles in flight while one is computed, plus one).
  // With the nontemporal tile loads, one buffer (no tile in flight during
  // the compute; the other wave of the SIMD overlaps it) ran fastest for
  // 2-byte caches on MI355X; the quantised tiles keep two.
#ifndef PKV_NBUF2B
#define PKV_NBUF2B 1
#endif
#ifndef PKV_NBUFQ
#define PKV_NBUFQ 2
#endif
  constexpr int NBUF = (DT == DT_F16 || DT == DT_BF16) ? PKV_NBUF2B : PKV_NBUFQ;
  static_assert(RB % 32 == 0 && CPR <= 64 && GP <= 16, "shape");
  static_assert(!Q4 || (NV == NP && BS % NV == 0), "q4_0 tile layout");
  // q4_0 and q8_0 at head_dim 128 with up to 4 heads per group: P.V on MFMA
  // (compute_tile); q8_0 there also takes q.K on fp16 MFMAs (Q8M).
  constexpr bool MPV = QN && D == 128 && GP <= 4;
  constexpr bool Q8M = Q8 && MPV;
  static_assert(!MPV || (CPR == 16 && NV == 4 && EPC == 8), "MFMA P.V lane layout");

  constexpr int NW = BINS ? kBinWaves : 1;  // waves per workgroup
  // softmax weights, [wave][row][head], then a spare slot the lanes without
  // a head write to (a store every lane makes needs no branch). One buffer
  // serves every tile: a wave's LDS operations complete in order, so the
  // next tile's writes cannot pass this tile's reads.
  __shared__ float p_lds_all[NW][16 * GP + 4];
  __shared__ float a_lds_all[NW][GP];          // per-head rescale factors
  __shared__ float l_lds_all[NW][GP];          // per-head sums at the end of a run
  __shared__ float m_lds_all[NW][GP];          // per-head maxima at the end of a run
  // BINS: pieces (o, m, l) of segments split between this workgroup's waves,
  // in the slots the host gives (a split segment's n pieces in n consecutive
  // slots; at most two pieces per wave)
  constexpr int NSLOT = NW * 2;
  __shared__ float piece_o[BINS ? NSLOT * GP * D : 1];
  __shared__ float piece_ml[BINS ? NSLOT * GP * 2 : 1];

  // the first nprefix workgroups (split form) take the shared-prefix items
  constexpr bool PFX = !BINS && D == 128 && (DT == DT_F16 || DT == DT_BF16);
  if constexpr (PFX) {
    if ((int)blockIdx.x < p.nprefix) {
      // Workgroups are dealt round-robin to the XCDs: XCD x takes items
      // [x * n / 8, (x + 1) * n / 8), which the host orders by kv head, so the
      // prompt tiles of a head are re-read from one XCD's L2.
      const int per = p.nprefix / kNumXcd;
      const int item = ((int)blockIdx.x % kNumXcd) * per + (int)blockIdx.x / kNumXcd;
      if (item < p.nitems) prefix_item<DT, GP, BS>(p, item);
      return;
    }
  }
  const int bid = (int)blockIdx.x - (PFX ? p.nprefix : 0);  // a multiple of 8 comes off
  // wave-uniform (scalar registers): the descriptor loads become scalar loads
  const int wl = BINS ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  const int lane = threadIdx.x & 63;
  float (&p_lds)[16 * GP + 4] = p_lds_all[wl];
  float (&a_lds)[GP] = a_lds_all[wl];
  float (&l_lds)[GP] = l_lds_all[wl];
  float (&m_lds)[GP] = m_lds_all[wl];
  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD one
  // contiguous eighth of the waves (bins) so neighbouring work shares an L2.
  const int wg = (bid % kNumXcd) * p.waves_per_xcd + bid / kNumXcd;
  const int w = BINS ? wg * NW + wl : wg;
  const bool active = w < p.nwaves;
  if (!BINS && !active) return;
#ifdef PKV_TIMELINE
  const long long tl_t0 = __builtin_amdgcn_s_memrealtime();
  long long tl_t1 = 0;
  int tl_tiles = 0, tl_segs = 0;
#endif

  // Per-wave descriptor: first tile (BINS: index of its first segment in the
  // bin lists), end tile (BINS: tile count), sequence, kv head, first block of
  // the run inside the sequence, context length, physical id of that block,
  // and (BINS) the merge it owns.
  const int* desc = p.wdesc + 8 * (active ? w : 0);
  int li = BINS ? desc[0] : 0;
  int x = BINS ? 0 : desc[0];
  const int xend = active ? desc[1] : 0;
  int s = desc[2];
  int g = desc[3];
  int j0 = desc[4];
  // context length; bit 30 set when the uploaded slot of the sequence is >= 0
  // (its new row is appended by a fused call)
  int L = desc[5] & kLenMask;
  int has_slot = desc[5] >> 30;
  int blk_first = desc[6];
  const int merge_info = BINS ? desc[7] : 0;
  // 8-token blocks: id of the block holding rows 8..15 of the run's first tile
  // (the split descriptor carries it; the bins form, whose descriptor word 7
  // is the merge, reads it from the table; any block when the context ends
  // before row 8)
  int blk_second = 0;
  if constexpr (!BINS) blk_second = desc[7];
  else if constexpr (BS == 8)
    blk_second = 16 * j0 + 8 < L ? p.bt[(size_t)s * p.bt_stride + 2 * j0 + 1] : blk_first;
  const int s_first = s, g_first = g;
  bool first_seg = true;
#ifdef PKV_TIMELINE
  // when the descriptor has arrived (the branch waits for it)
  const long long tl_td = uni(xend) < 0 ? 1 : __builtin_amdgcn_s_memrealtime();
#endif

  const int t16 = lane & 15;  // K row (token) this lane feeds; q row (head) likewise
  const int kg = lane >> 4;   // which 16-byte piece of each 64 bytes
  const bool head_lane = kg < NG;  // this lane's score rows are real heads
  const uint64_t head_mask = __builtin_amdgcn_ballot_w64(head_lane);
  const int vc = lane % CPR;  // V chunk this lane owns
  const int vr = lane / CPR;  // V row group of this lane
  // V row held in the lane's i-th chunk
  auto vrow = [&](int i) { return QN ? NV * vr + i : vr + RPI * i; };
  const size_t blk_stride = (size_t)p.kv_heads * TILE;

  while (x < xend) {
    const int nblk = (L + 15) >> 4;
    const int take = min(xend - x, nblk - j0);
    const int j1 = j0 + take;
    const int seg = g * p.batch + s;
    // Prefetch the next segment's length and first block id (vector loads in
    // flight while this segment's tiles stream; read as wave-uniform values at
    // the switch).
    int next_s = s + 1, next_g = g, next_L = 0, next_blk = 0, next_second = 0, next_j0 = 0;
    if constexpr (BINS) {
      if (x + take < xend) {  // bin lists hold (sequence, kv head, length, first block)
        const int* e = p.seglist + 4 * (li + 1);
        next_s = vld(e);
        next_g = vld(e + 1);
        next_L = vld(e + 2);
        next_blk = vld(e + 3);
        if constexpr (BS == 8)  // rows 8..15 of the first tile
          next_second = (next_L & kLenMask) > 8 ? vld(p.bt + (size_t)uni(next_s) * p.bt_stride + 1) : next_blk;
      }
    } else {
      if (next_s == p.batch) {
        next_s = 0;
        ++next_g;
      }
      if (x + take < xend) {
        next_L = vld(p.ctx + next_s);
        if (p.seqinfo) {
          // shared prefixes: the sequence's run starts at its first private
          // tile, whose block id(s) the host wrote beside it
          const int* r = p.seqinfo + 4 * next_s;
          next_j0 = vld(r);
          next_blk = vld(r + 1);
          next_second = vld(r + 2);
        } else {
          next_blk = vld(p.bt + (size_t)next_s * p.bt_stride);
          // 8-token blocks: the second entry (padding -1 when absent: any
          // block, its rows are past the context)
          if constexpr (BS == 8)
            next_second = p.bt_stride > 1 ? max(vld(p.bt + (size_t)next_s * p.bt_stride + 1), 0) : 0;
        }
      }
    }
    const char* kbase = reinterpret_cast<const char*>(p.k) + (size_t)g * TILE;
    const char* vbase = reinterpret_cast<const char*>(p.v) + (size_t)g * TILE;
    const int32_t* bt_row = p.bt + (size_t)s * p.bt_stride;

    // Append fused into the pass: the cached rows are ctx-1; the run holding
    // the last block also takes the new token's row from k_new / v_new as a
    // one-row tile, writes it to the pool where the table puts it and
    // attends over it.
    const bool app = p.k_new != nullptr && has_slot;
    const char* kn_row =
        reinterpret_cast<const char*>(p.k_new) + ((size_t)s * p.kv_heads + g) * QB;
    const char* vn_row =
        reinterpret_cast<const char*>(p.v_new) + ((size_t)s * p.kv_heads + g) * QB;
    const int Lc = L - (app ? 1 : 0);         // rows already in the pool
    const int j1c = min(j1, (Lc + 15) >> 4);  // tiles holding cached rows
    // q4_0 (groups of up to 4 heads): the run that ends the sequence requests
    // the new row now, beside the block-table entries, and appends it once
    // the first tile is on its way. Fetched and quantised at the end of the
    // run, it put a memory round trip (behind the run's own tile traffic) and
    // the quantising on the wave's critical path: 26 % of an 8B-shaped q4_0
    // layer, 12 % this way. The other caches keep the late form, which
    // measured faster for them (bf16 by 0.6 us, q8_0 by 1-1.5 us per layer:
    // the registers held early cost their loops more).
#ifndef PKV_EARLY_2B
#define PKV_EARLY_2B 0
#endif
    constexpr bool EARLY_NEW = (Q4 && GP <= 4) || (PKV_EARLY_2B && (DT == DT_F16 || DT == DT_BF16));
    const bool app_here = app && j1 == nblk;
    u32x4 nk[NP], nv = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < NP; ++k) nk[k] = u32x4{0u, 0u, 0u, 0u};
    if (EARLY_NEW && app_here) {
#pragma unroll
      for (int k = 0; k < NP; ++k) nk[k] = ld16(kn_row + kg * 16 + k * 64);
      nv = ld16(vn_row + vc * 16);
    }
    // the lane's K piece k and V chunk of the new row: requested early, or now
    auto new_k = [&](int k) { return EARLY_NEW ? nk[k] : ld16(kn_row + kg * 16 + k * 64); };
    auto new_v = [&]() { return EARLY_NEW ? nv : ld16(vn_row + vc * 16); };

    // Load tile rows 0..15 (tokens 16*j .. 16*j+15 of the sequence): block a
    // holds them (BS = 16), or rows 16*half .. of it (BS = 32), or rows 0..7
    // while block b holds rows 8..15 (BS = 8).
    auto load_tile = [&](int a, int b, int half, TR& t) {
      auto blk_of = [&](int r) { return BS == 8 ? (r < 8 ? a : b) : a; };
      auto rib = [&](int r) { return BS == 8 ? (r & 7) : BS == 32 ? 16 * half + r : r; };
      const char* ktile = kbase + (size_t)blk_of(t16) * blk_stride;
      const int kr = rib(t16);
      if constexpr (QN) {
        // piece k / chunk vc: codes 32*k + 8*kg .. +8 / 8*vc .. +8 of a row
        // the lane's NV consecutive V rows lie in one block
        const int r0 = NV * vr;
        const char* vtile = vbase + (size_t)blk_of(r0) * blk_stride;
        const int vrr = rib(r0);
        if constexpr (Q4) {
          // 4-byte words; the tile layout puts the lane's NP K words (one
          // quarter of row kr) and its NV V words (word vc of rows vrr ..
          // vrr+NV-1, NV = NP = groups per row) each in one contiguous run
          const char* kt = ktile + (unsigned)(kr * CB + kg * NP * 4);
          const char* vt = vtile + (unsigned)(vrr * CB + vc * NV * 4);
          if constexpr (NP == 4) {
            const u32x4 a = nt16(kt), b = nt16(vt);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              t.k[i] = a[i];
              t.v[i] = b[i];
            }
          } else {
            const u32x2 a = nt8(kt), b = nt8(vt);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              t.k[i] = a[i];
              t.v[i] = b[i];
            }
          }
        } else {
          // the layout puts the lane's pieces of groups 2c, 2c+1 (and its V
          // chunks of rows 2c, 2c+1 of its NV) as 16 bytes at c*R*64 +
          // lane*16 of the R-row part of the block (lane index within that
          // part): every load instruction reads R*64 contiguous bytes
          constexpr int R = BS < 16 ? BS : 16;
          const char* kt = ktile + (unsigned)((kr / R) * R * D + (kg * R + kr % R) * 16);
          const char* vt = vtile + (unsigned)((vrr / R) * R * D + ((vrr % R) / NV * CPR + vc) * 16);
#pragma unroll
          for (int c = 0; c < NP / 2; ++c) {
            const u32x4 a = nt16(kt + c * R * 64);
            t.k[2 * c] = u32x2{a[0], a[1]};
            t.k[2 * c + 1] = u32x2{a[2], a[3]};
          }
#pragma unroll
          for (int c = 0; c < NV / 2; ++c) {
            const u32x4 b = nt16(vt + c * R * 64);
            t.v[2 * c] = u32x2{b[0], b[1]};
            t.v[2 * c + 1] = u32x2{b[2], b[3]};
          }
        }
        // scales after the BS rows of codes: K [row][group], V [group][row]
        const char* ksp = ktile + (unsigned)(BS * CB + kr * NP * 2);
        const char* vsp = vtile + (unsigned)(BS * CB + ((vc >> 2) * BS + vrr) * 2);
        if constexpr (NP == 4) {
          const u32x2 x2 = ldsc8(ksp);
          t.ks[0] = x2[0];
          t.ks[1] = x2[1];
        } else {
          t.ks[0] = ldsc4(ksp);
        }
        if constexpr (NV == 4) {
          const u32x2 x2 = ldsc8(vsp);
          t.vs[0] = x2[0];
          t.vs[1] = x2[1];
        } else {
          t.vs[0] = ldsc4(vsp);
        }
      } else {
        const char* kt = ktile + kr * RB + kg * 16;
#pragma unroll
        for (int k = 0; k < NP; ++k) t.k[k] = nt16(kt + k * 64);
        if constexpr (BS == 8) {
          // row vr + RPI*i (vr < RPI, RPI divides 8) lies in block a iff RPI*i < 8
#pragma unroll
          for (int i = 0; i < NV; ++i)
            t.v[i] = nt16(vbase + (size_t)(RPI * i < 8 ? a : b) * blk_stride +
                          ((vr + RPI * i) & 7) * RB + vc * 16);
        } else {
          const char* vt = vbase + (size_t)a * blk_stride + rib(vr) * RB + vc * 16;
#pragma unroll
          for (int i = 0; i < NV; ++i) t.v[i] = nt16(vt + i * RPI * RB);
        }
      }
    };

    // q rows of the GQA group (row = head t16), in the same pieces as K. Rows
    // past the group repeat its last head: their scores land in rows no
    // output is taken from. Filled by setup_q once the run's first tile is
    // requested, so that its wait does not hold back that request.
    u32x4 qv[NP];
    // smul[i]: log2(e) x scale, times what turns score row i's MFMA result
    // into q . K (q8_0 and q4_0: the head's 2^(24 - qsh)).
    float smul[HPG];
    // The accumulator input of each piece's MFMA, from the scaled q piece's
    // sum over its group (an MFMA against ones): q4_0 -8 x 2^-24 times it,
    // turning q . code x 2^-24 into q . (code - 8) x 2^-24; q8_0 -128 x 2^-24
    // times it, for q . (128 + code) x 2^-24 into q . code x 2^-24.
    f32x4 qb[QN ? NP : 1];
    auto setup_q = [&]() {
    {
      const int hq = min(t16, p.group - 1);
      const char* qr = reinterpret_cast<const char*>(p.q) +
                       ((size_t)s * p.q_heads + (size_t)g * p.group + hq) * QB + kg * 16;
#pragma unroll
      for (int k = 0; k < NP; ++k) qv[k] = ld16(qr + k * 64);
    }
#pragma unroll
    for (int i = 0; i < HPG; ++i) smul[i] = p.scale_log2;
    if constexpr (Q4) {
      // q as fp16 in nibbles_to_f16's slot order (odd elements divided by
      // 16), each head scaled by the power of two 2^qsh that puts its
      // largest |q| in [2^14, 2^15): bf16's 8 significant bits are kept and
      // the products with the codes' 16c x 2^-24 stay far inside fp32.
      float qf[NP][8];
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        to_f32<DT_BF16>(qv[k], qf[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, __builtin_fabsf(qf[k][e]));
      }
      mx = fmaxf(mx, xor_f(mx, 16));
      mx = fmaxf(mx, xor_f(mx, 32));
      const int qsh = min(100, max(-100, 15 - __builtin_amdgcn_frexp_expf(mx)));
      const float f = __builtin_amdgcn_ldexpf(1.f, qsh), f16th = f * 0.0625f;
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const float* x = qf[k];
        qv[k][0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(x[0] * f, x[4] * f));
        qv[k][1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(x[1] * f16th, x[5] * f16th));
        qv[k][2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(x[2] * f, x[6] * f));
        qv[k][3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(x[3] * f16th, x[7] * f16th));
      }
#pragma unroll
      for (int i = 0; i < HPG; ++i)
        smul[i] = p.scale_log2 * __builtin_amdgcn_ldexpf(1.f, 24 - __shfl(qsh, 4 * kg + i, 64));
    }
    if constexpr (Q8M) {
      // q as fp16 for the MFMA against fp16 codes, each head scaled by 2^qsh
      // so that its largest |q| lies in [2^14, 2^15): no overflow, and bf16's
      // 8 significant bits are kept. Lanes t16, t16 + 16, +32, +48 hold head
      // t16's pieces.
      float qf[NP][8];
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        to_f32<DT_BF16>(qv[k], qf[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, __builtin_fabsf(qf[k][e]));
      }
      mx = fmaxf(mx, xor_f(mx, 16));
      mx = fmaxf(mx, xor_f(mx, 32));
      // mx = f 2^x with f in [0.5, 1) (x = 0 for 0); kept to a range where the
      // factors below stay finite
      const int qsh = min(100, max(-100, 15 - __builtin_amdgcn_frexp_expf(mx)));
      const float f = __builtin_amdgcn_ldexpf(1.f, qsh);
#pragma unroll
      for (int k = 0; k < NP; ++k)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          qv[k][w] = __builtin_bit_cast(
              unsigned, __builtin_amdgcn_cvt_pkrtz(qf[k][2 * w] * f, qf[k][2 * w + 1] * f));
#pragma unroll
      for (int i = 0; i < HPG; ++i)
        smul[i] = p.scale_log2 * __builtin_amdgcn_ldexpf(1.f, 24 - __shfl(qsh, 4 * kg + i, 64));
    }
    if constexpr (Q4) {
      // each head's scaled q piece summed (the slots' 1 or 16 undo the
      // division), times -8 x 2^-24: q . c x 2^-24 becomes q . (c - 8) x 2^-24
      const u32x4 ones = {0x3c003c00u, 0x4c004c00u, 0x3c003c00u, 0x4c004c00u};
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const f32x4 sq = qk_piece<DT_F16>(qv[k], ones, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) qb[k][i] = -0x1p-21f * sq[i];
      }
    } else if constexpr (Q8M) {
      const u32x4 ones = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const f32x4 sq = qk_piece<DT_F16>(qv[k], ones, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) qb[k][i] = -0x1p-17f * sq[i];
      }
    }
    };

    // Lane (t16, kg) keeps softmax state for heads 4*kg + i of its row.
    // mlz: m + kLazy, the score above which a tile raises the maxima
    float m[HPG], mlz[HPG], lsum[HPG];
    float acc[GP][EPC];
    float bsum[GP];  // q4_0: sum of the lane's scaled weights per head (8 x it is taken off)
    // MFMA P.V: block nt of output columns (head-dim columns 8 * n + nt), rows
    // 4 * (lane / 16) + i as the MFMA lays them out
    f32x4 accm[MPV ? 8 : 1];
#pragma unroll
    for (int nt = 0; nt < (MPV ? 8 : 1); ++nt) accm[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 accs = {0.f, 0.f, 0.f, 0.f};  // MFMA P.V: per row, the sum of its A values
#pragma unroll
    for (int i = 0; i < HPG; ++i) {
      m[i] = mlz[i] = -__builtin_inff();
      lsum[i] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      bsum[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
    }

    // A tile of valid < 16 rows (a segment's last) masks the rows past the
    // context, which may hold anything (NaN), in blocks that full tiles branch
    // around (valid is uniform across the wave): their scores become -inf and
    // their V values (q8_0 / q4_0: V scales) zero in the tile registers.
    // (The V registers are masked where V is first used, so that full tiles
    // do not wait for V before q.K.)
    // MFMA P.V: the A values (weight x V scale) and B operands of a tile
    // whose P.V waits for the next tile's, so that one MFMA 16x16x32 takes
    // the two tiles' high (then low) weight parts against their own codes.
    // bt[nt]: B operands of column block nt, the pending tile's in words 0-1
    // and the next tile's in words 2-3 (built in place).
    float pa_p[4];
    u32x4 bt[MPV ? 8 : 1];
    // one tile: its high and low weight parts against its codes twice
    auto pv_one = [&](const float (&pa)[4]) {
      if constexpr (MPV) {
        f16x4 h, l;
        split_f16(pa, h, l);
        const f16x8 av = {h[0], h[1], h[2], h[3], l[0], l[1], l[2], l[3]};
        accs = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, ones_f16(), accs, 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          bt[nt][2] = bt[nt][0];
          bt[nt][3] = bt[nt][1];
          accm[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(f16x8, bt[nt]),
                                                            accm[nt], 0, 0, 0);
        }
      }
    };
    auto compute_tile = [&](auto mode_tag, int valid, TR& t) {
      constexpr int MODE = MPV ? decltype(mode_tag)::value : 0;
      const bool part = __builtin_expect(valid < 16, 0);
      auto mask_v = [&]() {
        if (part) {
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            if (vrow(i) >= valid) {
              if constexpr (QN) t.vs[i >> 1] &= (i & 1) ? 0x0000ffffu : 0xffff0000u;
              else t.v[i] = u32x4{0u, 0u, 0u, 0u};
            }
          }
        }
      };
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (QN) {
        // one MFMA per 32-code group, then that group's scale for this
        // lane's token: sum_k d_k * (q_k . c_k)
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          f32x4 r;
          if constexpr (Q4) r = qk_piece<DT_F16>(qv[k], nibbles_to_f16(t.k[k]), qb[k]);
          else if constexpr (Q8M) r = qk_piece<DT_F16>(qv[k], codes_to_f16_128(t.k[k]), qb[k]);
          else r = qk_piece<DT_BF16>(qv[k], codes_to_bf16(t.k[k]), f32x4{0.f, 0.f, 0.f, 0.f});
          const float dk = (k & 1) ? half_hi(t.ks[k >> 1]) : half_lo(t.ks[k >> 1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[i] = __builtin_fmaf(dk, r[i], sacc[i]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NP; ++k) sacc = qk_piece<DT>(qv[k], t.k[k], sacc);
      }
      // sacc[i] = q(head 4*kg + i) . K(token t16)
      float s2[HPG];
      // MFMA P.V takes weight x scale as fp16: weights stay <= 2^kLazy, and a
      // tile with a V scale above 2^8 - 1 raises the maxima on any increase
      // (weights <= 1), so the products stay finite.
      bool big = false;
      if constexpr (MPV) {
        mask_v();
        // fp16 magnitude bits above 255 (0x5bf8), NaN included (rows past the
        // context may hold anything: that only costs a rescale)
        const unsigned a0 = t.vs[0] & 0x7fff7fffu, a1 = t.vs[1] & 0x7fff7fffu;
        const unsigned mx = max(max(a0 & 0xffffu, a0 >> 16), max(a1 & 0xffffu, a1 >> 16));
        big = wave_any(mx > 0x5bf8u);
      }
      // rows past the context (only a partial tile has them: in a full one
      // valid = 16) score -inf; a select, as such rows may hold anything
      const bool dead = t16 >= valid;
#pragma unroll
      for (int i = 0; i < HPG; ++i) s2[i] = dead ? -__builtin_inff() : sacc[i] * smul[i];
      // lanes with a score above its threshold, as wave masks (the compares'
      // own scalar results, OR-ed in scalar registers)
      uint64_t over = 0;
#pragma unroll
      for (int i = 0; i < HPG; ++i) over |= __builtin_amdgcn_ballot_w64(s2[i] > mlz[i]);
      if (big) {  // any increase
        over = 0;
#pragma unroll
        for (int i = 0; i < HPG; ++i) over |= __builtin_amdgcn_ballot_w64(s2[i] > m[i]);
      }
      if (over & head_mask) {  // raise the running maxima to this tile's
        float alpha[HPG];
#pragma unroll
        for (int i = 0; i < HPG; ++i) {
          // m - max(m, r) is min(m - r, 0) bit for bit; written so, the new
          // maximum replaces the old one in its register
          const float r = row_max(s2[i]);
          alpha[i] = __builtin_amdgcn_exp2f(fminf(m[i] - r, 0.f));
          m[i] = fmaxf(m[i], r);
          lsum[i] *= alpha[i];
          mlz[i] = m[i] + kLazy;
        }
        if (head_lane && t16 == 0) {
#pragma unroll
          for (int i = 0; i < HPG; ++i) a_lds[4 * kg + i] = alpha[i];
        }
        wave_sync();
        if constexpr (MPV) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = i < GP ? a_lds[i < GP ? i : 0] : 1.f;
            accs[i] *= a;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) accm[nt][i] *= a;
          }
          if constexpr (MODE == 2) {  // the pending tile's weights of head lane % 4
            const int hh = lane & 3;
            const float a = hh < GP ? a_lds[hh < GP ? hh : 0] : 1.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) pa_p[i] *= a;
          }
        } else {
#pragma unroll
          for (int h = 0; h < GP; ++h) {
            const float a = a_lds[h];
            bsum[h] *= a;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[h][e] *= a;
          }
        }
      }
      float* pl = p_lds;
      float* pw_at = pl + (head_lane ? t16 * GP + 4 * kg : 16 * GP);
#pragma unroll
      for (int i = 0; i < HPG; ++i) {
        const float pw = __builtin_amdgcn_exp2f(s2[i] - m[i]);
        lsum[i] += pw;
        pw_at[i] = pw;
      }
      wave_sync();
      if constexpr (MPV) {
        // P.V as MFMAs 16x16x32, one per block of 16 output columns and
        // weight part: A row 4 * G + h holds head h's weights times each
        // token's scale for group G (the spare rows of a group of <= 4 heads
        // carry the four scale groups), split into a high and a low fp16 part
        // (~22 bits together); k = the lane's 4 tokens of two tiles (or of one
        // tile twice, high and low parts side by side). B: column n of block
        // nt is head-dim column 8 * n + nt, its code's byte taken as the fp16
        // bits: the subnormal code x 2^-24 (odd nt: code x 2^-20), exact, and
        // kept by the MFMA. MFMAs against ones sum each row's A values, so the
        // 8 of code - 8 comes off at the end from the same fp16 parts. Row
        // 4 * G + h of block nt is head h's output for the columns of group
        // G, used by the lanes whose columns 8 * (lane % 16) + nt lie in
        // group lane / 16.
        const int hh = lane & 3;
        float pa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tr = 4 * vr + i;
          const float dv = (i & 1) ? half_hi(t.vs[i >> 1]) : half_lo(t.vs[i >> 1]);
          const float pw = pl[tr * GP + (hh < GP ? hh : 0)];
          pa[i] = hh < GP ? __builtin_fmaf(pw, dv, 0.f) : 0.f;
        }
        // this tile's B operands into words 0-1 (pending or alone) or 2-3
        constexpr int BW = MODE == 2 ? 2 : 0;
        if constexpr (Q8) {
          // 128 + code (the top bit flipped) of the 4 rows' chunks; column
          // 8 * n + nt is byte nt & 3 of word nt >> 2
          unsigned x[4][2];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int w = 0; w < 2; ++w) x[i][w] = t.v[i][w] ^ 0x80808080u;
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) {
            const int w = nt >> 2;
            const unsigned b = nt & 3;
            const unsigned sel = 0x0c000c00u | ((4u + b) << 16) | b;
            bt[nt][BW] = __builtin_amdgcn_perm(x[1][w], x[0][w], sel);
            bt[nt][BW + 1] = __builtin_amdgcn_perm(x[3][w], x[2][w], sel);
          }
        } else {
          unsigned ev[4], od[4];  // even codes (low nibbles), odd codes x 16 (high nibbles)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ev[i] = t.v[i] & 0x0f0f0f0fu;
            od[i] = t.v[i] & 0xf0f0f0f0u;
          }
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) {
            const unsigned* src = (nt & 1) ? od : ev;
            // byte nt / 2 of rows 0, 1 (and 2, 3) into the low bytes of the two fp16 halves
            const unsigned sel = 0x0c000c00u | ((4u + (nt >> 1)) << 16) | (unsigned)(nt >> 1);
            bt[nt][BW] = __builtin_amdgcn_perm(src[1], src[0], sel);
            bt[nt][BW + 1] = __builtin_amdgcn_perm(src[3], src[2], sel);
          }
        }
        if constexpr (MODE == 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) pa_p[i] = pa[i];
        } else if constexpr (MODE == 2) {
          f16x4 ah, al, bh, bl;
          split_f16(pa_p, ah, al);
          split_f16(pa, bh, bl);
          const f16x8 ahi = {ah[0], ah[1], ah[2], ah[3], bh[0], bh[1], bh[2], bh[3]};
          const f16x8 alo = {al[0], al[1], al[2], al[3], bl[0], bl[1], bl[2], bl[3]};
          accs = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, ones_f16(), accs, 0, 0, 0);
          accs = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, ones_f16(), accs, 0, 0, 0);
#pragma unroll
          for (int nt = 0; nt < 8; ++nt)
            accm[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, __builtin_bit_cast(f16x8, bt[nt]),
                                                              accm[nt], 0, 0, 0);
#pragma unroll
          for (int nt = 0; nt < 8; ++nt)
            accm[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, __builtin_bit_cast(f16x8, bt[nt]),
                                                              accm[nt], 0, 0, 0);
        } else {
          pv_one(pa);
        }
      } else {
      mask_v();
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int tr = vrow(i);
        float vals[EPC];
        float dv = 1.f;  // quantised: the row's scale for this lane's group
        if constexpr (QN) {
          code_vals(t.v[i], vals);
          dv = (i & 1) ? half_hi(t.vs[i >> 1]) : half_lo(t.vs[i >> 1]);
        } else {
          to_f32<DT>(t.v[i], vals);
        }
        float pt[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h) pt[h] = QN ? pl[tr * GP + h] * dv : pl[tr * GP + h];
        if constexpr (Q4) {
#pragma unroll
          for (int h = 0; h < GP; ++h) bsum[h] += pt[h];
        }
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][e] = __builtin_fmaf(pt[h], vals[e], acc[h][e]);
      }
      }
    };

    // Tile buffers; the chunk cursor, the block-table entries of the chunk
    // (one per lane) and the entry index of its first lane.
    TR t[NBUF];
    int jb = j0, nb = 0, my_ent = 0, e0_cur = -(1 << 30);
    // Tiles stream through NBUF register buffers: NBUF - 1 tiles are in
    // flight while one is computed. Block-table entries come one per lane, 64
    // at a time (the tiles of 64 entries: 64, 128 or 32 of them).
    constexpr int CH = BS == 8 ? 32 : 64;  // tiles per chunk of entries
    const int nent_seq = (L + BS - 1) / BS;
    // The new token: every lane takes the k_new / v_new row as row 0 of a
    // one-row tile (quantised in registers for q8_0 / q4_0, as the append
    // kernels do), the lanes of row 0 store it into the pool, and the tile is
    // attended. With the row requested early this runs at the start of the
    // run, while the first tile's loads are in flight (the pool row it writes
    // is masked out of that run's own last tile, and no other run reads it).
    auto append_new_row = [&]() {
      // the new row's block: from the entries of the last chunk requested
      // when they hold it, else from the table
      const int eidx = (L - 1) / BS;
      const int rel = eidx - e0_cur;
      const int blk_last = rel >= 0 && rel < 64 ? __builtin_amdgcn_readlane(my_ent, rel)
                                                : bt_row[eidx];
      const int t_new = (L - 1) % BS;  // the new row inside its block
      char* ktile = const_cast<char*>(kbase) + (size_t)blk_last * blk_stride;
      char* vtile = const_cast<char*>(vbase) + (size_t)blk_last * blk_stride;
      TR tn;
      if constexpr (Q4) {
        // As for q8_0 below, with the group's first largest-magnitude value
        // found across the same lanes and 4-bit codes.
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          float x[8];
          to_f32<DT_BF16>(new_k(k), x);
          float a, mv;
          int idx;
          q4_pick(x, 8 * kg, a, mv, idx);
          q4_pick_xor(a, mv, idx, 16);
          q4_pick_xor(a, mv, idx, 32);
          const float d = mv / -8.f;
          tn.k[k] = q4_codes(x, d);
          const unsigned hb = q4_scale_bits(mv, d);
          if (k & 1) tn.ks[k >> 1] |= hb << 16;
          else tn.ks[k >> 1] = hb;
        }
        {
          float x[8];
          to_f32<DT_BF16>(new_v(), x);
          float a, mv;
          int idx;
          q4_pick(x, 8 * (vc & 3), a, mv, idx);
          q4_pick_xor(a, mv, idx, 1);
          q4_pick_xor(a, mv, idx, 2);
          const float d = mv / -8.f;
          const unsigned c = q4_codes(x, d);
#pragma unroll
          for (int i = 0; i < NV; ++i) tn.v[i] = c;  // only row 0 is attended
#pragma unroll
          for (int i = 0; i < NV / 2; ++i) tn.vs[i] = 0u;
          tn.vs[0] = q4_scale_bits(mv, d);
          if (vr == 0) {
            *reinterpret_cast<unsigned*>(vtile + (t_new - t_new % NV) * CB +
                                         (vc * NV + t_new % NV) * 4) = c;
            if ((vc & 3) == 0)
              *reinterpret_cast<unsigned short*>(vtile + BS * CB + ((vc >> 2) * BS + t_new) * 2) =
                  (unsigned short)tn.vs[0];
          }
        }
        if (t16 == 0) {
          char* kw = ktile + t_new * CB + kg * NP * 4;  // the lane's NP words, contiguous
          if constexpr (NP == 4) *reinterpret_cast<u32x4*>(kw) = u32x4{tn.k[0], tn.k[1], tn.k[2], tn.k[3]};
          else *reinterpret_cast<u32x2*>(kw) = u32x2{tn.k[0], tn.k[1]};
          if (kg == 0) {
            char* ksp = ktile + BS * CB + t_new * NP * 2;
            if constexpr (NP == 4) *reinterpret_cast<u32x2*>(ksp) = u32x2{tn.ks[0], tn.ks[1]};
            else *reinterpret_cast<unsigned*>(ksp) = tn.ks[0];
          }
        }
      } else if constexpr (Q8) {
        // Quantise the bf16 row group by group (as the append kernel does):
        // K group k is spread over the four lanes kg of a token column, a V
        // group over four neighbouring chunks of one row.
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          float x[8];
          to_f32<DT_BF16>(new_k(k), x);
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) a = fmaxf(a, __builtin_fabsf(x[j]));
          a = fmaxf(a, xor_f(a, 16));
          a = fmaxf(a, xor_f(a, 32));
          float d;
          tn.k[k] = q8_codes(x, a, &d);
          const unsigned hb = half_bits(d);
          if (k & 1) tn.ks[k >> 1] |= hb << 16;
          else tn.ks[k >> 1] = hb;
        }
        {
          float x[8];
          to_f32<DT_BF16>(new_v(), x);
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) a = fmaxf(a, __builtin_fabsf(x[j]));
          a = fmaxf(a, xor_f(a, 1));
          a = fmaxf(a, xor_f(a, 2));
          float d;
          const u32x2 c = q8_codes(x, a, &d);
#pragma unroll
          for (int i = 0; i < NV; ++i) tn.v[i] = c;  // only row 0 is attended
#pragma unroll
          for (int i = 0; i < NV / 2; ++i) tn.vs[i] = 0u;
          tn.vs[0] = half_bits(d);
          if (vr == 0) {
            *reinterpret_cast<u32x2*>(vtile + q8_chunk_offset<D>(true, t_new, vc, BS)) = c;
            if ((vc & 3) == 0)
              *reinterpret_cast<unsigned short*>(vtile + BS * D + ((vc >> 2) * BS + t_new) * 2) =
                  (unsigned short)tn.vs[0];
          }
        }
        if (t16 == 0) {
#pragma unroll
          for (int k = 0; k < NP; ++k)
            *reinterpret_cast<u32x2*>(ktile + q8_chunk_offset<D>(false, t_new, 4 * k + kg, BS)) =
                tn.k[k];
          if (kg == 0) {
            char* ksp = ktile + BS * D + t_new * NP * 2;
            if constexpr (NP == 4) *reinterpret_cast<u32x2*>(ksp) = u32x2{tn.ks[0], tn.ks[1]};
            else *reinterpret_cast<unsigned*>(ksp) = tn.ks[0];
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < NP; ++k) tn.k[k] = new_k(k);
#pragma unroll
        for (int i = 0; i < NV; ++i) tn.v[i] = new_v();
        if (t16 == 0) {
#pragma unroll
          for (int k = 0; k < NP; ++k)
            *reinterpret_cast<u32x4*>(ktile + t_new * RB + kg * 16 + k * 64) = tn.k[k];
        }
        if (vr == 0) *reinterpret_cast<u32x4*>(vtile + t_new * RB + vc * 16) = tn.v[0];
      }
      compute_tile(PvMode<0>{}, 1, tn);
    };
    // block ids of chunk tile j: (a, b, half)
    auto tile_ids = [&](int j, int& a, int& b, int& half) {
      if constexpr (BS == 16) {
        a = b = __builtin_amdgcn_readlane(my_ent, j);
        half = 0;
      } else if constexpr (BS == 32) {
        a = b = __builtin_amdgcn_readlane(my_ent, ((jb + j) >> 1) - (jb >> 1));
        half = (jb + j) & 1;
      } else {
        a = __builtin_amdgcn_readlane(my_ent, 2 * j);
        b = __builtin_amdgcn_readlane(my_ent, 2 * j + 1);
        half = 0;
      }
    };
    auto load_j = [&](int j, TR& t) {
      int a, b, half;
      tile_ids(j, a, b, half);
      load_tile(a, b, half, t);
    };
    // Block-table entries first, one per lane (up to 64: CH tiles need CH
    // (16), 2 * CH = 64 (8) or CH / 2 + 1 (32)), then the first tile, whose
    // id(s) the descriptor holds for the run's first chunk: the first wait
    // for the entries then leaves that tile's loads in flight.
    auto start_chunk = [&]() {
      nb = min(CH, j1c - jb);
      const int e0 = BS == 32 ? (jb >> 1) : BS == 8 ? 2 * jb : jb;
      my_ent = e0 + lane < nent_seq ? bt_row[e0 + lane] : 0;
      e0_cur = e0;
      if (jb == j0) load_tile(blk_first, BS == 8 ? blk_second : 0, BS == 32 ? (jb & 1) : 0, t[0]);
      else load_j(0, t[0]);
#pragma unroll
      for (int u = 1; u < NBUF - 1; ++u) load_j(min(u, nb - 1), t[u]);
    };
    // the first chunk's entries and first tile are requested before q
    if (jb < j1c) start_chunk();
    setup_q();
    if (EARLY_NEW && app_here) append_new_row();
    for (; jb < j1c; jb += CH) {
      if (jb != j0) start_chunk();
      // Every step requests a tile, the chunk's last one again once the chunk
      // is exhausted (a repeat the cache serves): with no conditional loads
      // the compiler's wait counts stay static and only the tile about to be
      // computed is waited for, never the one just requested.
      for (int jj = 0; jj < nb; jj += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          const int j = jj + u;
          if (j < nb) {
            // one buffer: tile 0 of the chunk was requested by start_chunk
            if constexpr (NBUF > 1) load_j(min(j + NBUF - 1, nb - 1), t[(u + NBUF - 1) % NBUF]);
            else if (j > 0) load_j(j, t[0]);
            // keep the scheduler from hoisting the compute (and its waits) above
            // the request
            __builtin_amdgcn_sched_barrier(0);
            const int valid = min(16, Lc - 16 * (jb + j));
            if constexpr (MPV && NBUF == 2) {
              // P.V of tile pairs (the pair's first tile waits)
              if (u == 0) compute_tile(PvMode<1>{}, valid, t[u]);
              else compute_tile(PvMode<2>{}, valid, t[u]);
            } else {
              compute_tile(PvMode<0>{}, valid, t[u]);
            }
#ifdef PKV_TIMELINE
            if (tl_t1 == 0) tl_t1 = __builtin_amdgcn_s_memrealtime();
            ++tl_tiles;
#endif
          }
        }
      }
    }
    if constexpr (MPV && NBUF == 2) {
      // Every chunk but the run's last has an even tile count (CH is even),
      // so a tile is left pending only at the end of a run of odd length.
      static_assert(CH % 2 == 0, "tile pairs within chunks");
      if (j1c > j0 && ((j1c - j0) & 1)) pv_one(pa_p);
    }
    if (!EARLY_NEW && app_here) append_new_row();

    // Totals over the 16 rows, and over the lanes sharing a V chunk.
    float lt[HPG];
#pragma unroll
    for (int i = 0; i < HPG; ++i) lt[i] = row_sum(lsum[i]);
    if constexpr (MPV) {
      // the MFMA summed over the tile's rows: sum A x code x 2^-24 (q4_0's
      // odd columns 2^-20), less 8 x sum A (q8_0: 128 + code, less 128 x sum A)
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          acc[h][e] = Q8 ? __builtin_fmaf(accm[e][h], 16777216.f, -128.f * accs[h])
                         : __builtin_fmaf(accm[e][h], (e & 1) ? 1048576.f : 16777216.f,
                                          -8.f * accs[h]);
    } else {
      if constexpr (Q4) {  // sum_t w_t (code_t - 8) = sum_t w_t code_t - 8 sum_t w_t
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][e] = __builtin_fmaf(-8.f, bsum[h], acc[h][e]);
      }
#pragma unroll
      for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][e] += xor_f(acc[h][e], off);
    }
    // lanes holding the output: columns pv_col .. pv_col + EPC - 1 of every head
    const bool pv_lane = MPV ? (lane >> 4) == ((lane & 15) >> 2) : lane < CPR;
    const int pv_col = (MPV ? (lane & 15) : lane) * EPC;
    if (head_lane && t16 == 0) {
#pragma unroll
      for (int i = 0; i < HPG; ++i) {
        l_lds[4 * kg + i] = lt[i];
        m_lds[4 * kg + i] = m[i];
      }
    }
    wave_sync();
    const bool whole = j0 == 0 && j1 == nblk;
    if (whole) {
      if (pv_lane) {
        float* o = p.out + ((size_t)s * p.q_heads + (size_t)g * p.group) * D + pv_col;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if (h < p.group) {
            const float inv = 1.f / l_lds[h];
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[(size_t)h * D + e] = acc[h][e] * inv;
          }
        }
      }
    } else if constexpr (BINS) {
      const int slot = first_seg ? (merge_info & 15) : ((merge_info >> 4) & 15);
      float* po = piece_o + (size_t)(slot * GP) * D + pv_col;
      if (pv_lane) {
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
          for (int e = 0; e < EPC; ++e) po[(size_t)h * D + e] = acc[h][e];
      }
      if (lane < p.group) {
        piece_ml[(slot * GP + lane) * 2 + 0] = m_lds[lane];
        piece_ml[(slot * GP + lane) * 2 + 1] = l_lds[lane];
      }
    } else {
      // slots of segment seg: ((seg + 1) * stride - 1) + its waves; the
      // stride - 1 slots before them hold its shared-prefix partials
      const size_t idx = (size_t)(seg + 1) * p.seg_stride - 1 + w;
      if (pv_lane) {
        float* o = p.part_o + idx * GP * D + pv_col;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if (h < p.group) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[(size_t)h * D + e] = acc[h][e];
          }
        }
      }
      if (lane < p.group) {
        p.part_ml[(idx * GP + lane) * 2 + 0] = m_lds[lane];
        p.part_ml[(idx * GP + lane) * 2 + 1] = l_lds[lane];
      }
    }
    wave_sync();  // l_lds / m_lds / a_lds are reused by the next run

#ifdef PKV_TIMELINE
    ++tl_segs;
#endif
    x += take;
    if (x >= xend) break;
    s = uni(next_s);
    g = uni(next_g);
    j0 = uni(next_j0);
    L = uni(next_L) & kLenMask;
    has_slot = uni(next_L) >> 30;
    blk_first = uni(next_blk);
    blk_second = uni(next_second);
    ++li;
    first_seg = false;
  }

#ifdef PKV_TIMELINE
  const long long tl_t2 = __builtin_amdgcn_s_memrealtime();
  long long tl_tb = 0;
#endif
  if constexpr (BINS) {
    // Every piece of this bin is in LDS: each segment split between waves is
    // merged head by head by the waves holding its pieces (slot 0 of each,
    // except the first holder's, whose slot the host gives):
    //   out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
    // Only LDS is exchanged: the barrier orders LDS alone and does not wait
    // for this wave's global stores (outputs, appended rows) to complete.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#ifdef PKV_TIMELINE
    tl_tb = __builtin_amdgcn_s_memrealtime();
#endif
    // Head hh of a segment whose n pieces are in slots base .. base+n-1. All
    // LDS reads are issued before the arithmetic: every lane reads each
    // piece's max and sum (the same words in every lane) and its D/64 columns
    // of every piece, and weighs the pieces itself (no cross-lane steps).
    auto merge_head = [&](int ms, int mg, int base, int n, int hh) {
      constexpr int PER = D / 64;
      float mm[NW], ll[NW], src[NW][PER];
      const float* mlp = piece_ml + (base * GP + hh) * 2;
      const float* op = piece_o + (size_t)(base * GP + hh) * D + lane * PER;
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        if (k < n) {
          mm[k] = mlp[k * GP * 2];
          ll[k] = mlp[k * GP * 2 + 1];
#pragma unroll
          for (int e = 0; e < PER; ++e) src[k][e] = op[(size_t)k * GP * D + e];
        }
      }
      float M = mm[0];
#pragma unroll
      for (int k = 1; k < NW; ++k)
        if (k < n) M = fmaxf(M, mm[k]);
      float den = 0.f, o[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        if (k < n) {
          const float wv = __builtin_amdgcn_exp2f(mm[k] - M);
          den = __builtin_fmaf(wv, ll[k], den);
#pragma unroll
          for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(wv, src[k][e], o[e]);
        }
      }
      const float inv = __builtin_amdgcn_rcpf(den);
      float* dst =
          p.out + ((size_t)ms * p.q_heads + (size_t)mg * p.group + hh) * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) dst[e] = o[e] * inv;
    };
    if (active && (merge_info & (1 << 8))) {
      // this wave's first segment: n pieces from slot base, this wave the
      // idx-th holder; it merges heads idx, idx + n, ...
      const int base = (merge_info >> 9) & 15, n = (merge_info >> 13) & 15;
      for (int hh = (merge_info >> 17) & 7; hh < p.group; hh += n)
        merge_head(s_first, g_first, base, n, hh);
    }
    if (active && (merge_info & (1 << 20))) {
      // this wave's last segment: started here, its n pieces from this
      // wave's slot on
      const int base = (merge_info >> 4) & 15, n = (merge_info >> 21) & 15;
      for (int hh = 0; hh < p.group; hh += n) merge_head(s, g, base, n, hh);
    }
  }
#ifdef PKV_TIMELINE
  if (active && lane == 0 && w < 8192) {
    long long* r = pkv_tl + 8 * w;
    r[6] = tl_tb;
    r[7] = tl_td;
    r[0] = tl_t0;
    r[1] = tl_t1;
    r[2] = tl_t2;
    r[3] = __builtin_amdgcn_s_memrealtime();
    r[4] = (__builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xf) | (tl_tiles << 8) |
           ((long long)tl_segs << 24);
    r[5] = w;
  }
#endif
}

// Segments with many partials (a long context at a fixed split): one
// workgroup of four waves per (sequence, q head). Each wave takes every
// fourth group of partials, a lane 4 columns of one partial (lanes past the
// first D/4 the next partials); up to 4 * PPW * U partials are loaded at once,
// with their (m, l), and M comes from those registers (a block reduction),
// so the merge waits on memory once; more partials take a first pass for M
// and then U groups of loads at a time. The waves' sums meet in LDS:
//   out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
template <int D, int GP>
__global__ __launch_bounds__(256) void reduce_wide_kernel(ReduceParams p) {
  constexpr int LPP = D / 4;     // lanes per partial (4 columns each)
  constexpr int PPW = 64 / LPP;  // partials per wave per load step
  constexpr int U = 32;          // load steps in flight
  constexpr int STEP = 4 * PPW * U;
  __shared__ float red[4];
  __shared__ float osum[4 * PPW][D];
  __shared__ float dsum[4 * PPW];
  const int pair = blockIdx.x;  // one (sequence, q head) per workgroup
  const int s = pair / p.q_heads;
  const int h = pair % p.q_heads;
  const int g = h / p.group;
  const int hh = h - g * p.group;
  const int seg = g * p.batch + s;
  const int w0 = p.seg_w0[seg];
  const int w1 = p.seg_w1[seg];
  const int npre = p.seqinfo ? p.seqinfo[4 * s + 3] : 0;
  if (w0 == w1 && npre == 0) return;  // written directly by the decode kernel
  const size_t first = (size_t)(seg + 1) * p.seg_stride - 1 + w0 - npre;
  const int n = w1 - w0 + 1 + npre;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* ml = p.part_ml + (first * GP + hh) * 2;  // partial i at ml[i * GP * 2]
  const int sub = lane / LPP, col = (lane % LPP) * 4;
  const float* po = p.part_o + (first * GP + hh) * D + col;  // partial i at po[i * GP * D]
  auto block_max = [&](float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, xor_f(x, off));
    if (lane == 0) red[wave] = x;
    __syncthreads();
    x = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();  // red is written again only after every wave has read it
    return x;
  };
  float o[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
  float M = -__builtin_inff();
  if (n > STEP) {
    for (int i = tid; i < n; i += 256) M = fmaxf(M, ml[(size_t)i * GP * 2]);
    M = block_max(M);
  }
  for (int base = 0; base < n; base += STEP) {
    float4 v[U];
    float mm[U], ll[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + (u * 4 + wave) * PPW + sub;
      const bool ok = i < n;
      v[u] = ok ? *reinterpret_cast<const float4*>(po + (size_t)i * GP * D)
                : float4{0.f, 0.f, 0.f, 0.f};
      mm[u] = ok ? ml[(size_t)i * GP * 2] : -__builtin_inff();
      ll[u] = ok ? ml[(size_t)i * GP * 2 + 1] : 0.f;
    }
    if (n <= STEP) {  // every partial is in registers: M from them
#pragma unroll
      for (int u = 0; u < U; ++u) M = fmaxf(M, mm[u]);
      M = block_max(M);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = mm[u] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mm[u] - M);
      den = __builtin_fmaf(w, ll[u], den);
      o[0] = __builtin_fmaf(w, v[u].x, o[0]);
      o[1] = __builtin_fmaf(w, v[u].y, o[1]);
      o[2] = __builtin_fmaf(w, v[u].z, o[2]);
      o[3] = __builtin_fmaf(w, v[u].w, o[3]);
    }
  }
  const int slot = wave * PPW + sub;
#pragma unroll
  for (int e = 0; e < 4; ++e) osum[slot][col + e] = o[e];
  if (lane % LPP == 0) dsum[slot] = den;
  __syncthreads();
  if (tid < D) {
    float acc = 0.f, dd = 0.f;
#pragma unroll
    for (int k = 0; k < 4 * PPW; ++k) {
      acc += osum[k][tid];
      dd += dsum[k];
    }
    p.out[((size_t)s * p.q_heads + h) * D + tid] = acc * __builtin_amdgcn_rcpf(dd);
  }
}

// Four wavefronts per workgroup, one (sequence, q head) pair each: fewer,
// larger workgroups keep the dispatch ramp of this short kernel small.
template <int D, int GP>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams p) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= p.batch * p.q_heads) return;
  const int s = pair / p.q_heads;
  const int h = pair % p.q_heads;
  const int g = h / p.group;
  const int hh = h - g * p.group;
  const int seg = g * p.batch + s;
  const int w0 = p.seg_w0[seg];
  const int w1 = p.seg_w1[seg];
  // shared-prefix chunks: partials in the slots just before the run's own
  const int npre = p.seqinfo ? p.seqinfo[4 * s + 3] : 0;
  if (w0 == w1 && npre == 0) return;  // written directly by the decode kernel
  merge_partials<D, GP>(p.part_o, p.part_ml, (size_t)(seg + 1) * p.seg_stride - 1 + w0 - npre,
                        w1 - w0 + 1 + npre, hh, p.out + ((size_t)s * p.q_heads + h) * D, lane);
}

// Appends skip a slot outside [0, num_slots) (num_blocks * block_size): a
// stale or bad slot from the caller never becomes a store outside the pool.
// Workgroups in row order, nslice per new row (each 256 of its (K|V, kv
// head, 16-byte chunk) pieces, one per thread; the row's slot is one scalar
// load). Row bytes and block sizes are powers of two, so every index below
// the row is a shift or a mask. The new rows are read once and the pool rows
// written once: nontemporal accesses stream both past the caches.
__global__ __launch_bounds__(256) void append_kernel(const char* k_new, const char* v_new,
                                                     const int64_t* slots, char* k_layer,
                                                     char* v_layer, int kv_heads, int row_shift,
                                                     int bs_shift, int nslice, int64_t num_slots) {
  const unsigned bid = blockIdx.x;
  const unsigned row = bid / (unsigned)nslice;
  const size_t s = row;
  const int64_t slot = slots[s];
  if (slot < 0 || slot >= num_slots) return;
  const int cshift = row_shift - 4;  // 16-byte chunks per row: 1 << cshift
  const int t = (int)(bid - row * (unsigned)nslice) * 256 + (int)threadIdx.x;
  const int chunk = t & ((1 << cshift) - 1);
  const int r = t >> cshift;
  const int kv = r & 1, g = r >> 1;
  if (g >= kv_heads) return;
  const size_t blk = (size_t)(slot >> bs_shift);
  const size_t pos = (size_t)(slot & ((1 << bs_shift) - 1));
  const char* src = (kv ? v_new : k_new) + ((s * kv_heads + g) << row_shift) + chunk * 16;
  char* dst = (kv ? v_layer : k_layer) +
              ((((blk * kv_heads + g) << bs_shift) + pos) << row_shift) + chunk * 16;
  __builtin_nontemporal_store(nt16(src), reinterpret_cast<u32x4*>(dst));
}

// Thread of the quantised appends -> (32-value group, K or V, kv head, row of
// the batch): the group fastest, then 16 consecutive rows, then K/V and the
// head. The tile layouts spread one row's codes over several lines that
// neighbouring rows fill too, so a wave writing 16 consecutive rows of a
// multi-token write covers whole lines instead of pieces of them.
struct QuantAppendItem {
  int grp, kv, g, s;
};
// 32-bit thread indices (the launcher checks the count), ngr a power of two.
__device__ __forceinline__ QuantAppendItem quant_append_item(unsigned idx, int ngr,
                                                             unsigned kv_heads) {
  QuantAppendItem it;
  it.grp = (int)(idx & (unsigned)(ngr - 1));
  unsigned t = idx / (unsigned)ngr;
  const int rr = (int)(t & 15);
  t >>= 4;
  it.kv = (int)(t & 1);
  t >>= 1;
  const unsigned q = t / kv_heads;
  it.g = (int)(t - q * kv_heads);
  it.s = (int)(q * 16 + rr);
  return it;
}

// q8_0 append: one thread per (sequence, kv head, K|V, 32-value group) of
// the bf16 new rows; writes 32 codes into the row and the group's fp16 scale
// (K scales [row][group], V scales [group][row] after the tile's codes).
template <int D>
__global__ __launch_bounds__(256) void append_q8_kernel(const char* k_new, const char* v_new,
                                                        const int64_t* slots, int batch,
                                                        char* k_layer, char* v_layer,
                                                        int kv_heads, int block_size,
                                                        int64_t num_slots) {
  constexpr int NGR = D / 32;
  const int BS = block_size;
  const int TILE = BS * D + BS * NGR * 2;
  const QuantAppendItem it =
      quant_append_item(blockIdx.x * 256u + threadIdx.x, NGR, (unsigned)kv_heads);
  const int grp = it.grp, kv = it.kv, g = it.g;
  const int s = it.s;
  if (s >= batch) return;
  const int64_t slot = slots[s];
  if (slot < 0 || slot >= num_slots) return;
  const int bs_shift = __builtin_ctz((unsigned)BS);  // block sizes are powers of two
  const int64_t blk = slot >> bs_shift;
  const int pos = (int)(slot & (BS - 1));
  const char* src = (kv ? v_new : k_new) + (((size_t)s * kv_heads + g) * D + grp * 32) * 2;
  float x[4][8];
  float a = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    to_f32<DT_BF16>(ld16(src + c * 16), x[c]);
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, __builtin_fabsf(x[c][j]));
  }
  char* tile = (kv ? v_layer : k_layer) + ((size_t)blk * kv_heads + g) * TILE;
  float d = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)  // the group's four chunks of 8 codes
    *reinterpret_cast<u32x2*>(tile + q8_chunk_offset<D>(kv, pos, 4 * grp + c, BS)) =
        q8_codes(x[c], a, &d);
  const int si = kv ? grp * BS + pos : pos * NGR + grp;
  *reinterpret_cast<unsigned short*>(tile + BS * D + si * 2) = (unsigned short)half_bits(d);
}

// q4_0 append: as append_q8_kernel, with the group's first largest-magnitude
// value m, scale m / -8 and 16 bytes of packed 4-bit codes per group.
template <int D>
__global__ __launch_bounds__(256) void append_q4_kernel(const char* k_new, const char* v_new,
                                                        const int64_t* slots, int batch,
                                                        char* k_layer, char* v_layer,
                                                        int kv_heads, int block_size,
                                                        int64_t num_slots) {
  constexpr int NGR = D / 32;
  constexpr int CB = D / 2;
  const int BS = block_size;
  const int TILE = BS * CB + BS * NGR * 2;
  const QuantAppendItem it =
      quant_append_item(blockIdx.x * 256u + threadIdx.x, NGR, (unsigned)kv_heads);
  const int grp = it.grp, kv = it.kv, g = it.g;
  const int s = it.s;
  if (s >= batch) return;
  const int64_t slot = slots[s];
  if (slot < 0 || slot >= num_slots) return;
  const int bs_shift = __builtin_ctz((unsigned)BS);  // block sizes are powers of two
  const int64_t blk = slot >> bs_shift;
  const int pos = (int)(slot & (BS - 1));
  const char* src = (kv ? v_new : k_new) + (((size_t)s * kv_heads + g) * D + grp * 32) * 2;
  float x[4][8];
  float a = 0.f, m = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    to_f32<DT_BF16>(ld16(src + c * 16), x[c]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float ax = __builtin_fabsf(x[c][j]);
      if (ax > a) {
        a = ax;
        m = x[c][j];
      }
    }
  }
  const float d = m / -8.f;
  char* tile = (kv ? v_layer : k_layer) + ((size_t)blk * kv_heads + g) * TILE;
  // word w = 4 * grp + c of the row (elements 8w .. 8w+7): K words transposed
  // within the row, V rows interleaved NGR at a time
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int wd = 4 * grp + c;
    const int off = kv ? (pos - pos % NGR) * CB + (wd * NGR + pos % NGR) * 4
                       : pos * CB + (c * NGR + grp) * 4;
    *reinterpret_cast<unsigned*>(tile + off) = q4_codes(x[c], d);
  }
  const int si = kv ? grp * BS + pos : pos * NGR + grp;
  *reinterpret_cast<unsigned short*>(tile + BS * CB + si * 2) = (unsigned short)q4_scale_bits(m, d);
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(const int32_t* pairs, int layers,
                                                          char* k_base, char* v_base,
                                                          int64_t layer_bytes,
                                                          int64_t block_bytes) {
  const int per_pair = layers * 2;
  const int pair = blockIdx.x / per_pair;
  const int rem = blockIdx.x % per_pair;
  const int layer = rem >> 1;
  const int kv = rem & 1;
  const int64_t src = pairs[2 * pair];
  const int64_t dst = pairs[2 * pair + 1];
  char* base = (kv ? v_base : k_base) + layer * layer_bytes;
  const char* sp = base + src * block_bytes;
  char* dp = base + dst * block_bytes;
  for (int64_t off = (int64_t)threadIdx.x * 16; off < block_bytes; off += 256 * 16)
    *reinterpret_cast<u32x4*>(dp + off) = *reinterpret_cast<const u32x4*>(sp + off);
}

// Pinned host memory (read over PCIe) -> device, 16 bytes per lane, grid-stride.
__global__ __launch_bounds__(256) void upload_kernel(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// The bins form is built for 16-token blocks only.
template <int DT, int D, int GP, int BS>
const void* decode_fn_bs(bool bins) {
  if (!bins) return reinterpret_cast<const void*>(&decode_kernel<DT, D, GP, false, BS>);
  if constexpr (DT == DT_F32) return nullptr;  // fp32 tiles spill in the eight-wave form
  else return reinterpret_cast<const void*>(&decode_kernel<DT, D, GP, true, BS>);
}

template <int DT, int D, int GP>
const void* decode_fn(bool bins, int bs) {
  switch (bs) {
    case 8: return decode_fn_bs<DT, D, GP, 8>(bins);
    case 16: return decode_fn_bs<DT, D, GP, 16>(bins);
    case 32: return decode_fn_bs<DT, D, GP, 32>(bins);
  }
  return nullptr;
}

template <int DT, int D>
const void* pick_gp(int gp, bool bins, int bs) {
  switch (gp) {
    case 1: return decode_fn<DT, D, 1>(bins, bs);
    case 2: return decode_fn<DT, D, 2>(bins, bs);
    case 4: return decode_fn<DT, D, 4>(bins, bs);
    case 8: return decode_fn<DT, D, 8>(bins, bs);
  }
  return nullptr;
}

template <int DT>
const void* pick_d(int d, int gp, bool bins, int bs) {
  switch (d) {
    case 64: return pick_gp<DT, 64>(gp, bins, bs);
    case 128: return pick_gp<DT, 128>(gp, bins, bs);
  }
  return nullptr;
}

const void* decode_kernel_for(int dtype, int d, int gp, bool bins, int bs) {
  switch (dtype) {
    case DT_F32: return pick_d<DT_F32>(d, gp, bins, bs);
    case DT_F16: return pick_d<DT_F16>(d, gp, bins, bs);
    case DT_BF16: return pick_d<DT_BF16>(d, gp, bins, bs);
    case DT_Q8: return pick_d<DT_Q8>(d, gp, bins, bs);
    case DT_Q4: return pick_d<DT_Q4>(d, gp, bins, bs);
  }
  return nullptr;
}

template <int D>
const void* reduce_for_gp(int gp, bool wide) {
  switch (gp) {
    case 1: return wide ? reinterpret_cast<const void*>(&reduce_wide_kernel<D, 1>)
                        : reinterpret_cast<const void*>(&reduce_kernel<D, 1>);
    case 2: return wide ? reinterpret_cast<const void*>(&reduce_wide_kernel<D, 2>)
                        : reinterpret_cast<const void*>(&reduce_kernel<D, 2>);
    case 4: return wide ? reinterpret_cast<const void*>(&reduce_wide_kernel<D, 4>)
                        : reinterpret_cast<const void*>(&reduce_kernel<D, 4>);
    case 8: return wide ? reinterpret_cast<const void*>(&reduce_wide_kernel<D, 8>)
                        : reinterpret_cast<const void*>(&reduce_kernel<D, 8>);
  }
  return nullptr;
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, int gp, bool bins, int block_size,
                         const DecodeParams& p, hipStream_t stream) {
  const void* fn = decode_kernel_for(dtype, head_dim, gp, bins, block_size);
  if (!fn) return hipErrorInvalidValue;
  DecodeParams args = p;
  void* argv[] = {&args};
  dim3 grid((unsigned)(p.nprefix + p.waves_per_xcd * kNumXcd)), block(bins ? 64 * kBinWaves : 64);
  return hipLaunchKernel(fn, grid, block, argv, 0, stream);
}

int decode_blocks_per_cu(int dtype, int head_dim, int gp, bool bins, int block_size) {
  const void* fn = decode_kernel_for(dtype, head_dim, gp, bins, block_size);
  if (!fn) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, bins ? 64 * kBinWaves : 64, 0) != hipSuccess)
    return 0;
  return n;
}

hipError_t launch_reduce(int head_dim, int gp, const ReduceParams& p, bool wide,
                         hipStream_t stream) {
  const void* fn = head_dim == 64 ? reduce_for_gp<64>(gp, wide)
                   : head_dim == 128 ? reduce_for_gp<128>(gp, wide) : nullptr;
  if (!fn) return hipErrorInvalidValue;
  ReduceParams args = p;
  void* argv[] = {&args};
  const unsigned pairs = (unsigned)(p.batch * p.q_heads);
  dim3 grid(wide ? pairs : (pairs + 3) / 4), block(256);
  return hipLaunchKernel(fn, grid, block, argv, 0, stream);
}

bool prefix_supported(int dtype, int head_dim, int gp) {
  return (dtype == DT_F16 || dtype == DT_BF16) && head_dim == 128 &&
         (gp == 1 || gp == 2 || gp == 4 || gp == 8);
}

hipError_t launch_append(const void* k_new, const void* v_new, const int64_t* slots, int batch,
                         void* k_layer, void* v_layer, int kv_heads, int row_bytes,
                         int block_size, int64_t num_slots, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  if (row_bytes < 16 || block_size < 1) return hipErrorInvalidValue;
  const int row_shift = __builtin_ctz((unsigned)row_bytes);
  const int bs_shift = __builtin_ctz((unsigned)block_size);
  if ((1 << row_shift) != row_bytes || (1 << bs_shift) != block_size) return hipErrorInvalidValue;
  const int pieces = 2 * kv_heads * (row_bytes / 16);  // per new row
  const int nslice = (pieces + 255) / 256;
  if ((int64_t)batch * nslice > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)(batch * nslice)), dim3(256), 0, stream,
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), slots,
                     static_cast<char*>(k_layer), static_cast<char*>(v_layer), kv_heads,
                     row_shift, bs_shift, nslice, num_slots);
  return hipGetLastError();
}

hipError_t launch_append_quant(int dtype, const void* k_new, const void* v_new,
                               const int64_t* slots, int batch, void* k_layer, void* v_layer,
                               int kv_heads, int head_dim, int block_size, int64_t num_slots,
                               hipStream_t stream) {
  // rows in groups of 16 (quant_append_item); the padding rows' threads return
  if (batch <= 0) return hipSuccess;
  const long threads = (long)((batch + 15) / 16) * 16 * kv_heads * 2 * (head_dim / 32);
  if (threads > 0xffffff00L) return hipErrorInvalidValue;  // 32-bit thread indices
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const char* kn = static_cast<const char*>(k_new);
  const char* vn = static_cast<const char*>(v_new);
  char* kl = static_cast<char*>(k_layer);
  char* vl = static_cast<char*>(v_layer);
  void (*fn)(const char*, const char*, const int64_t*, int, char*, char*, int, int, int64_t) =
      nullptr;
  if (dtype == DT_Q8) fn = head_dim == 128 ? append_q8_kernel<128>
                           : head_dim == 64 ? append_q8_kernel<64> : nullptr;
  if (dtype == DT_Q4) fn = head_dim == 128 ? append_q4_kernel<128>
                           : head_dim == 64 ? append_q4_kernel<64> : nullptr;
  if (!fn) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, grid, block, 0, stream, kn, vn, slots, batch, kl, vl, kv_heads,
                     block_size, num_slots);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const int32_t* pairs, int n, void* k_base, void* v_base,
                              int layers, int64_t layer_bytes, int64_t block_bytes,
                              hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)(n * layers * 2)), dim3(256), 0, stream,
                     pairs, layers, static_cast<char*>(k_base), static_cast<char*>(v_base),
                     layer_bytes, block_bytes);
  return hipGetLastError();
}

hipError_t launch_upload(const void* host_src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t wg = n16 < 256 * 256 ? (n16 + 255) / 256 : 256;
  hipLaunchKernelGGL(upload_kernel, dim3((unsigned)wg), dim3(256), 0, stream,
                     static_cast<const u32x4*>(host_src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

// Scratch for the split partials of the allocation-free decode. Host code
// never uses this name as an address: the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(int dev, void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev) return hipErrorInvalidDevice;  // the device must be current
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

#ifdef PKV_TIMELINE
hipError_t copy_timeline(void* dst, size_t bytes) {
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(pkv_tl), bytes < sizeof(pkv_tl) ? bytes : sizeof(pkv_tl), 0,
                             hipMemcpyDeviceToHost);
}
#endif

}  // namespace pkv
