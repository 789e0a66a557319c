// HIP kernels for paged KV-cache decode on MI355X (gfx950, wave64).
//
//  decode_kernel  — per wavefront: a contiguous run of (kv head, sequence,
//                   block) tiles; gathers 16 x head_dim K and V tiles through
//                   the block table with 128-bit loads, computes q.K^T for all
//                   query heads of the GQA group sharing the kv head, keeps an
//                   fp32 online softmax and accumulates P.V. A run that covers a
//                   whole (kv head, sequence) writes the normalised output;
//                   otherwise it writes an unnormalised partial (max, sum, o).
//  reduce_kernel  — merges the partials of one (sequence, q head):
//                   out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i.
//  append_kernel  — scatters each sequence's new K/V rows into the pool at its slot.
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
// full 16-byte lanes, and all arithmetic is plain fp32 VALU work.
#include "pkv_internal.h"

namespace pkv {
namespace {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct Elem {
  static constexpr int bytes = DT == DT_F32 ? 4 : 2;
};

__device__ __forceinline__ u32x4 ld16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Bit casts from one 32-bit lane of a u32x4. The element is copied to a
// scalar first: __builtin_bit_cast applied directly to a vector element
// expression reads element 0 whatever the index.
template <typename T>
__device__ __forceinline__ T lane_as(u32x4 v, int i) {
  const unsigned u = v[i];
  return __builtin_bit_cast(T, u);
}

// Dot product of one 16-byte piece of q with the matching piece of a K row,
// accumulated in fp32. bf16/fp16 products are exact in fp32; the dot2
// instructions add two of them per step.
template <int DT>
__device__ __forceinline__ float dot_piece(u32x4 q, u32x4 k, float acc) {
  if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(lane_as<bf16x2>(q, i), lane_as<bf16x2>(k, i), acc,
                                            false);
  } else if constexpr (DT == DT_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(lane_as<f16x2>(q, i), lane_as<f16x2>(k, i), acc, false);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_fmaf(lane_as<float>(q, i), lane_as<float>(k, i), acc);
  }
  return acc;
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

// Lanes 4r..4r+3 hold partial dot products of one K row for GP heads.
// Sum them within the quad. With GP >= 4 the sums are scattered so lane
// (4r + q) keeps heads q, q+4, ...; with GP < 4 every lane keeps all heads.
template <int GP>
__device__ __forceinline__ void quad_reduce(const float (&sc)[GP],
                                            float (&out)[GP >= 4 ? GP / 4 : GP], int lane) {
  if constexpr (GP >= 4) {
    const bool b1 = lane & 2;
    float k1[GP / 2];
#pragma unroll
    for (int i = 0; i < GP / 2; ++i) {
      const int h0 = (i / 2) * 4 + (i % 2);  // heads with bit 1 clear
      const int h1 = h0 + 2;
      const float keep = b1 ? sc[h1] : sc[h0];
      const float send = b1 ? sc[h0] : sc[h1];
      k1[i] = keep + xor_f(send, 2);
    }
    const bool b0 = lane & 1;
#pragma unroll
    for (int i = 0; i < GP / 4; ++i) {
      const float keep = b0 ? k1[2 * i + 1] : k1[2 * i];
      const float send = b0 ? k1[2 * i] : k1[2 * i + 1];
      out[i] = keep + xor_f(send, 1);
    }
  } else {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float v = sc[h];
      v += xor_f(v, 2);
      v += xor_f(v, 1);
      out[h] = v;
    }
  }
}

template <int DT, int D, int GP>
__global__ __launch_bounds__(64) void decode_kernel(DecodeParams p) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int RB = D * EB;       // bytes per K/V row
  constexpr int NP = RB / 64;      // 16-byte K pieces per lane per tile (4 lanes per row)
  constexpr int CPR = RB / 16;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;    // rows covered by one V load instruction
  constexpr int NV = 16 / RPI;     // V loads per lane per tile
  constexpr int EPC = 16 / EB;     // elements per chunk
  constexpr int HPL = GP >= 4 ? GP / 4 : GP;  // heads whose scores a lane holds
  constexpr int TILE = 16 * RB;
  static_assert(RB % 64 == 0 && CPR <= 64, "row size");

  __shared__ float p_lds[16 * GP];  // softmax weights of the current tile, [row][head]
  __shared__ float a_lds[GP];       // per-head rescale factor of the current tile
  __shared__ float l_lds[GP];       // per-head sums at the end of a run
  __shared__ float m_lds[GP];       // per-head maxima at the end of a run

  const int lane = threadIdx.x;
  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD one
  // contiguous eighth of the tile space so a kv head's tiles share one L2.
  const int w = (blockIdx.x % kNumXcd) * p.waves_per_xcd + blockIdx.x / kNumXcd;
  if (w >= p.nwaves) return;
  int x = p.wave_start[w];
  const int xend = p.wave_start[w + 1];
  if (x >= xend) return;

  const int row = lane >> 2;        // K row this lane's quad reads
  const int quad = lane & 3;
  const int vc = lane % CPR;        // V chunk this lane owns
  const int vr = lane / CPR;        // first V row of this lane

  // Locate the first tile: kv head, then sequence (count of prefix sums <= r).
  int g = x / p.tseq;
  int s;
  {
    const int r = x - g * p.tseq;
    int cnt = 0;
    for (int base = 0; base <= p.batch; base += 64) {
      const int i = base + lane;
      const int v = i <= p.batch ? p.cum[i] : 0x7fffffff;
      cnt += __popcll(__ballot(v <= r));
    }
    s = cnt - 1;
  }

  while (x < xend) {
    const int L = p.ctx[s];
    const int nblk = (L + 15) >> 4;
    const int j0 = x - g * p.tseq - p.cum[s];
    const int take = min(xend - x, nblk - j0);
    const int j1 = j0 + take;

    // q of the GQA group, in this lane's K pieces; padded heads are zero.
    u32x4 qv[GP][NP];
    {
      const char* qb = reinterpret_cast<const char*>(p.q) +
                       ((size_t)s * p.q_heads + (size_t)g * p.group) * RB;
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int k = 0; k < NP; ++k)
          qv[h][k] = h < p.group ? ld16(qb + (size_t)h * RB + (quad + 4 * k) * 16)
                                 : u32x4{0u, 0u, 0u, 0u};
    }

    float m[HPL], lsum[HPL];
    float acc[GP][EPC];
#pragma unroll
    for (int i = 0; i < HPL; ++i) {
      m[i] = -__builtin_inff();
      lsum[i] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;

    const int32_t* bt_row = p.bt + (size_t)s * p.bt_stride;
    const char* kbase = reinterpret_cast<const char*>(p.k) + (size_t)g * TILE;
    const char* vbase = reinterpret_cast<const char*>(p.v) + (size_t)g * TILE;
    const size_t blk_stride = (size_t)p.kv_heads * TILE;

    auto load_tile = [&](int blk, u32x4 (&kb)[NP], u32x4 (&vb)[NV]) {
      const char* kt = kbase + (size_t)blk * blk_stride + row * RB + quad * 16;
      const char* vt = vbase + (size_t)blk * blk_stride + vr * RB + vc * 16;
#pragma unroll
      for (int k = 0; k < NP; ++k) kb[k] = ld16(kt + k * 64);
#pragma unroll
      for (int i = 0; i < NV; ++i) vb[i] = ld16(vt + i * RPI * RB);
    };

    auto compute_tile = [&](int j, const u32x4 (&kb)[NP], const u32x4 (&vb)[NV]) {
      const int valid = min(16, L - 16 * j);
      float sc[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < NP; ++k) a = dot_piece<DT>(qv[h][k], kb[k], a);
        sc[h] = a;
      }
      float s2[HPL];
      quad_reduce<GP>(sc, s2, lane);
      float mt[HPL];
#pragma unroll
      for (int i = 0; i < HPL; ++i) {
        s2[i] = row < valid ? s2[i] * p.scale_log2 : -__builtin_inff();
        mt[i] = s2[i];
      }
#pragma unroll
      for (int off = 4; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < HPL; ++i) mt[i] = fmaxf(mt[i], xor_f(mt[i], off));
      bool changed = false;
      float alpha[HPL], pw[HPL];
#pragma unroll
      for (int i = 0; i < HPL; ++i) {
        const float mn = fmaxf(m[i], mt[i]);
        changed |= mn != m[i];
        alpha[i] = __builtin_amdgcn_exp2f(m[i] - mn);
        pw[i] = __builtin_amdgcn_exp2f(s2[i] - mn);
        lsum[i] = lsum[i] * alpha[i] + pw[i];
        m[i] = mn;
      }
      __syncthreads();  // previous tile's reads of p_lds/a_lds are done
      if constexpr (GP >= 4) {
#pragma unroll
        for (int i = 0; i < HPL; ++i) {
          p_lds[row * GP + 4 * i + quad] = pw[i];
          if (row == 0) a_lds[4 * i + quad] = alpha[i];
        }
      } else {
        if (quad == 0) {
#pragma unroll
          for (int i = 0; i < HPL; ++i) {
            p_lds[row * GP + i] = pw[i];
            if (row == 0) a_lds[i] = alpha[i];
          }
        }
      }
      __syncthreads();
      if (__any(changed)) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          const float a = a_lds[h];
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][e] *= a;
        }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int t = vr + RPI * i;
        float vals[EPC];
        to_f32<DT>(vb[i], vals);
        if (t >= valid) {  // rows past the context may hold anything (NaN)
#pragma unroll
          for (int e = 0; e < EPC; ++e) vals[e] = 0.f;
        }
        float pt[GP];
#pragma unroll
        for (int h = 0; h < GP; ++h) pt[h] = p_lds[t * GP + h];
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][e] = __builtin_fmaf(pt[h], vals[e], acc[h][e]);
      }
    };

    for (int jb = j0; jb < j1; jb += 64) {
      const int nb = min(64, j1 - jb);
      const int my_blk = lane < nb ? bt_row[jb + lane] : 0;
      u32x4 ka[NP], va[NV], kb2[NP], vb2[NV];
      load_tile(__builtin_amdgcn_readlane(my_blk, 0), ka, va);
      for (int jj = 0; jj < nb; jj += 2) {
        if (jj + 1 < nb) load_tile(__builtin_amdgcn_readlane(my_blk, jj + 1), kb2, vb2);
        compute_tile(jb + jj, ka, va);
        if (jj + 1 < nb) {
          if (jj + 2 < nb) load_tile(__builtin_amdgcn_readlane(my_blk, jj + 2), ka, va);
          compute_tile(jb + jj + 1, kb2, vb2);
        }
      }
    }

    // Totals over the 16 rows, and over the lanes sharing a V chunk.
    float lt[HPL];
#pragma unroll
    for (int i = 0; i < HPL; ++i) {
      float v = lsum[i];
#pragma unroll
      for (int off = 4; off < 64; off <<= 1) v += xor_f(v, off);
      lt[i] = v;
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] += xor_f(acc[h][e], off);
    __syncthreads();
    if constexpr (GP >= 4) {
      if (row == 0) {
#pragma unroll
        for (int i = 0; i < HPL; ++i) {
          l_lds[4 * i + quad] = lt[i];
          m_lds[4 * i + quad] = m[i];
        }
      }
    } else {
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < HPL; ++i) {
          l_lds[i] = lt[i];
          m_lds[i] = m[i];
        }
      }
    }
    __syncthreads();
    if (lane < CPR) {
      const bool whole = j0 == 0 && j1 == nblk;
      if (whole) {
        float* o = p.out + ((size_t)s * p.q_heads + (size_t)g * p.group) * D + lane * EPC;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if (h < p.group) {
            const float inv = 1.f / l_lds[h];
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[(size_t)h * D + e] = acc[h][e] * inv;
          }
        }
      } else {
        const size_t idx = (size_t)g * p.batch + s + w;
        float* o = p.part_o + idx * GP * D + lane * EPC;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if (h < p.group) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[(size_t)h * D + e] = acc[h][e];
            if (lane == 0) {
              p.part_ml[(idx * GP + h) * 2 + 0] = m_lds[h];
              p.part_ml[(idx * GP + h) * 2 + 1] = l_lds[h];
            }
          }
        }
      }
    }

    x += take;
    if (++s == p.batch) {
      s = 0;
      ++g;
    }
  }
}

template <int D, int GP>
__global__ __launch_bounds__(64) void reduce_kernel(ReduceParams p) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int s = blockIdx.x / p.q_heads;
  const int h = blockIdx.x % p.q_heads;
  const int g = h / p.group;
  const int hh = h - g * p.group;
  const int seg = g * p.batch + s;
  const int w0 = p.seg_w0[seg];
  const int w1 = p.seg_w1[seg];
  if (w0 == w1) return;  // written directly by the decode kernel
  const int n = w1 - w0 + 1;
  const size_t base = (size_t)seg + w0;

  float M = -__builtin_inff();
  for (int i = lane; i < n; i += 64) M = fmaxf(M, p.part_ml[((base + i) * GP + hh) * 2]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, xor_f(M, off));
  float den = 0.f;
  for (int i = lane; i < n; i += 64) {
    const float* ml = p.part_ml + ((base + i) * GP + hh) * 2;
    den += __builtin_amdgcn_exp2f(ml[0] - M) * ml[1];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) den += xor_f(den, off);

  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int i = 0; i < n; ++i) {
    const float wgt = __builtin_amdgcn_exp2f(p.part_ml[((base + i) * GP + hh) * 2] - M);
    const float* src = p.part_o + ((base + i) * GP + hh) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(wgt, src[e], o[e]);
  }
  const float inv = 1.f / den;
  float* dst = p.out + ((size_t)s * p.q_heads + h) * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[e] = o[e] * inv;
}

__global__ __launch_bounds__(256) void append_kernel(const char* k_new, const char* v_new,
                                                     const int64_t* slots, int batch,
                                                     char* k_layer, char* v_layer, int kv_heads,
                                                     int row_bytes) {
  const int per_row = row_bytes / 16;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int chunk = (int)(idx % per_row);
  long r = idx / per_row;
  const int kv = (int)(r & 1);
  r >>= 1;
  const int g = (int)(r % kv_heads);
  const long s = r / kv_heads;
  if (s >= batch) return;
  const int64_t slot = slots[s];
  if (slot < 0) return;
  const int64_t blk = slot >> 4;
  const int64_t pos = slot & 15;
  const char* src = (kv ? v_new : k_new) + ((size_t)s * kv_heads + g) * row_bytes + chunk * 16;
  char* dst = (kv ? v_layer : k_layer) + (((size_t)blk * kv_heads + g) * 16 + pos) * row_bytes +
              chunk * 16;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
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

template <int DT, int D, int GP>
const void* decode_fn() {
  return reinterpret_cast<const void*>(&decode_kernel<DT, D, GP>);
}

template <int DT, int D>
const void* pick_gp(int gp) {
  switch (gp) {
    case 1: return decode_fn<DT, D, 1>();
    case 2: return decode_fn<DT, D, 2>();
    case 4: return decode_fn<DT, D, 4>();
    case 8: return decode_fn<DT, D, 8>();
  }
  return nullptr;
}

template <int DT>
const void* pick_d(int d, int gp) {
  switch (d) {
    case 64: return pick_gp<DT, 64>(gp);
    case 128: return pick_gp<DT, 128>(gp);
  }
  return nullptr;
}

const void* decode_kernel_for(int dtype, int d, int gp) {
  switch (dtype) {
    case DT_F32: return pick_d<DT_F32>(d, gp);
    case DT_F16: return pick_d<DT_F16>(d, gp);
    case DT_BF16: return pick_d<DT_BF16>(d, gp);
  }
  return nullptr;
}

template <int D>
const void* reduce_for_gp(int gp) {
  switch (gp) {
    case 1: return reinterpret_cast<const void*>(&reduce_kernel<D, 1>);
    case 2: return reinterpret_cast<const void*>(&reduce_kernel<D, 2>);
    case 4: return reinterpret_cast<const void*>(&reduce_kernel<D, 4>);
    case 8: return reinterpret_cast<const void*>(&reduce_kernel<D, 8>);
  }
  return nullptr;
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, int gp, const DecodeParams& p,
                         hipStream_t stream) {
  const void* fn = decode_kernel_for(dtype, head_dim, gp);
  if (!fn) return hipErrorInvalidValue;
  DecodeParams args = p;
  void* argv[] = {&args};
  dim3 grid((unsigned)(p.waves_per_xcd * kNumXcd)), block(64);
  return hipLaunchKernel(fn, grid, block, argv, 0, stream);
}

int decode_blocks_per_cu(int dtype, int head_dim, int gp) {
  const void* fn = decode_kernel_for(dtype, head_dim, gp);
  if (!fn) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 64, 0) != hipSuccess) return 0;
  return n;
}

hipError_t launch_reduce(int head_dim, int gp, const ReduceParams& p, hipStream_t stream) {
  const void* fn = head_dim == 64 ? reduce_for_gp<64>(gp)
                   : head_dim == 128 ? reduce_for_gp<128>(gp) : nullptr;
  if (!fn) return hipErrorInvalidValue;
  ReduceParams args = p;
  void* argv[] = {&args};
  dim3 grid((unsigned)(p.batch * p.q_heads)), block(64);
  return hipLaunchKernel(fn, grid, block, argv, 0, stream);
}

hipError_t launch_append(const void* k_new, const void* v_new, const int64_t* slots, int batch,
                         void* k_layer, void* v_layer, int kv_heads, int row_bytes,
                         hipStream_t stream) {
  const long threads = (long)batch * kv_heads * 2 * (row_bytes / 16);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), slots,
                     batch, static_cast<char*>(k_layer), static_cast<char*>(v_layer), kv_heads,
                     row_bytes);
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

}  // namespace pkv
