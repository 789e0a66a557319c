// Bandwidth probes: measurements that bound the decode from above, not part of
// the decode path. Both read with the 16-byte nontemporal loads the decode
// uses for its K/V tiles and do no arithmetic beyond an XOR of what they read
// (one word per lane is written, so no load is dead).
//   stream: a contiguous buffer, each wave reading one contiguous share.
//   gather: every K and V tile the decode of one layer reads (16 tokens of
//     one kv head of one sequence), through the uploaded block table, the
//     (kv head, sequence, tile) space split into equal shares, one per wave:
//     the decode's access pattern with perfect balance and no compute.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned pu32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ pu32x4 ntl(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const pu32x4*>(p));
}

constexpr int kProbeWaves = 4;  // waves per workgroup

__global__ __launch_bounds__(64 * kProbeWaves) void probe_stream_kernel(const char* buf,
                                                                       int64_t n16, int nw,
                                                                       unsigned* out) {
  const int w = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= nw) return;
  const int64_t per = (n16 + nw - 1) / nw;  // 16-byte pieces per wave
  const int64_t a = (int64_t)w * per, e = a + per < n16 ? a + per : n16;
  pu32x4 x = {0u, 0u, 0u, 0u};
  int64_t i = a + lane;
  // eight loads of 1 KiB per wave in flight, then their XOR
  for (; i + 7 * 64 < e; i += 8 * 64) {
    pu32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ntl(buf + 16 * (i + 64 * k));
#pragma unroll
    for (int k = 0; k < 8; ++k) x ^= v[k];
  }
  for (; i < e; i += 64) x ^= ntl(buf + 16 * i);
  out[(int64_t)w * 64 + lane] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// NPL: 16-byte pieces per lane per tile (tile bytes / 1024).
template <int NPL>
__global__ __launch_bounds__(64 * kProbeWaves) void probe_gather_kernel(GatherParams p) {
  const int w = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= p.nwaves) return;
  const int64_t tseq = p.cum[p.batch];
  const int64_t T = tseq * p.kv_heads;
  int64_t x = T * w / p.nwaves;
  const int64_t xend = T * (w + 1) / p.nwaves;
  pu32x4 acc = {0u, 0u, 0u, 0u};
  if (x < xend) {
    // (kv head, sequence, tile) of the first tile: binary search in the
    // tiles' prefix sums
    int g = (int)(x / tseq);
    const int64_t r = x - (int64_t)g * tseq;
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cum[mid] <= r) lo = mid;
      else hi = mid - 1;
    }
    int s = lo;
    int j = (int)(r - p.cum[s]);
    int nblk = p.cum[s + 1] - p.cum[s];
    // block ids 64 at a time, one per lane
    int e0 = j, ent = j + lane < nblk ? p.bt[(int64_t)s * p.bt_stride + j + lane] : 0;
    pu32x4 cur[2 * NPL], nxt[2 * NPL];
    auto load = [&](int blk, pu32x4 (&t)[2 * NPL]) {
      const char* kt = p.k + (int64_t)blk * p.blk_stride + (int64_t)g * p.tile;
      const char* vt = p.v + (int64_t)blk * p.blk_stride + (int64_t)g * p.tile;
#pragma unroll
      for (int c = 0; c < NPL; ++c) {
        t[c] = ntl(kt + 16 * (lane + 64 * c));
        t[NPL + c] = ntl(vt + 16 * (lane + 64 * c));
      }
    };
    auto advance = [&]() {
      if (++j == nblk) {
        j = 0;
        if (++s == p.batch) {
          s = 0;
          ++g;
        }
        nblk = p.cum[s + 1] - p.cum[s];
        e0 = 0;
        ent = lane < nblk ? p.bt[(int64_t)s * p.bt_stride + lane] : 0;
      } else if (j - e0 == 64) {
        e0 = j;
        ent = j + lane < nblk ? p.bt[(int64_t)s * p.bt_stride + j + lane] : 0;
      }
    };
    load(__builtin_amdgcn_readlane(ent, j - e0), cur);
    for (++x; x < xend; ++x) {
      advance();
      load(__builtin_amdgcn_readlane(ent, j - e0), nxt);  // the next tile in flight
#pragma unroll
      for (int c = 0; c < 2 * NPL; ++c) acc ^= cur[c];
#pragma unroll
      for (int c = 0; c < 2 * NPL; ++c) cur[c] = nxt[c];
    }
#pragma unroll
    for (int c = 0; c < 2 * NPL; ++c) acc ^= cur[c];
  }
  p.out[(int64_t)w * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

hipError_t launch_probe_stream(const void* buf, int64_t bytes, int nwaves, unsigned* out,
                               hipStream_t stream) {
  const int grid = (nwaves + kProbeWaves - 1) / kProbeWaves;
  hipLaunchKernelGGL(probe_stream_kernel, dim3(grid), dim3(64 * kProbeWaves), 0, stream,
                     static_cast<const char*>(buf), bytes / 16, nwaves, out);
  return hipGetLastError();
}

hipError_t launch_probe_gather(const GatherParams& p, hipStream_t stream) {
  const int grid = (p.nwaves + kProbeWaves - 1) / kProbeWaves;
  switch (p.tile) {
    case 1024: hipLaunchKernelGGL(probe_gather_kernel<1>, dim3(grid), dim3(64 * kProbeWaves), 0, stream, p); break;
    case 2048: hipLaunchKernelGGL(probe_gather_kernel<2>, dim3(grid), dim3(64 * kProbeWaves), 0, stream, p); break;
    case 4096: hipLaunchKernelGGL(probe_gather_kernel<4>, dim3(grid), dim3(64 * kProbeWaves), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
