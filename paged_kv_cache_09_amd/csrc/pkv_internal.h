// Internal interface between the host library (pkv_host.cpp) and the HIP
// kernels (pkv_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kTile = 16;        // tokens per decode tile (a block of 16, half of 32, two of 8)
constexpr int kMaxGroup = 8;     // largest GQA group (q heads per kv head)
constexpr int kNumXcd = 8;       // MI355X: workgroups are dealt round-robin to 8 XCDs
#ifndef PKV_BIN_WAVES
#define PKV_BIN_WAVES 8
#endif
constexpr int kBinWaves = PKV_BIN_WAVES;  // waves per workgroup (bin) of the bins form

struct DecodeParams {
  const void* k;               // layer base of K: [num_blocks][kv_heads][16][head_dim]
  const void* v;               // layer base of V, same shape
  const int32_t* bt;           // block table [batch][bt_stride]
  const int32_t* ctx;          // context lengths [batch]
  const int32_t* wdesc;        // per wave: x0, x1, seq, kv head, j0, ctx, first block, 0
  const int32_t* seg_w0;       // first wave touching each (kv head, sequence) segment
  const int32_t* seg_w1;       // last wave touching it
  const int32_t* seglist;      // bins form: per listed segment (sequence, kv head, length,
                               // first block id), bins one after another
  const void* q;               // [batch][q_heads][head_dim], cache dtype
  const void* k_new;           // null, or new K rows [batch][kv_heads][head_dim] to append
  const void* v_new;           // new V rows (with k_new)
  const int64_t* slots;        // uploaded slots (with k_new): < 0 skips a sequence
  float* out;                  // [batch][q_heads][head_dim]
  float* part_o;               // [(nseg + nwaves) * gp][head_dim] unnormalised partial outputs
  float* part_ml;              // [(nseg + nwaves) * gp][2] partial (max, sum), log2 domain
  float scale_log2;            // softmax scale * log2(e)
  int32_t bt_stride;
  int32_t batch;
  int32_t kv_heads;
  int32_t q_heads;
  int32_t group;               // q_heads / kv_heads
  int32_t nwaves;
  int32_t waves_per_xcd;       // ceil(nwaves / 8)
  // shared prefixes (split form): null, or per sequence [first private tile,
  // its block id, (8-token blocks) the id of its rows 8..15, prefix chunks]
  const int32_t* seqinfo;
  int32_t seg_stride;          // partial slots per segment: 1 + most prefix chunks
  const int32_t* items;        // shared-prefix work items [nitems][kItemInts]
  const int32_t* groups;       // their groups [ngroups][kGroupInts]
  int32_t nitems;
  int32_t nprefix;             // leading workgroups for the items (multiple of 8)
};

struct ReduceParams {
  const float* part_o;
  const float* part_ml;
  const int32_t* seg_w0;       // first wave touching each (kv head, sequence) segment
  const int32_t* seg_w1;       // last wave touching it
  float* out;
  int32_t batch;
  int32_t kv_heads;
  int32_t q_heads;
  int32_t group;
  const int32_t* seqinfo;      // as in DecodeParams
  int32_t seg_stride;
};

// Shared-prefix items: tiles that a group of sequences reads from the same
// blocks (their common prompt), read once per group.
constexpr int kGroupInts = 20;   // per group: count, leader, chunks, 17 member slots
constexpr int kMaxMembers = 16;  // MFMA rows / padded heads per kv head
constexpr int kItemInts = 8;     // per work item: group, kv head, t0, t1, chunk, 0, 0, 0


// Padded group size used by the kernels: 1, 2, 4 or 8.
inline int padded_group(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : 8; }

// bins: the eight-wave form that merges split segments in LDS (waves_per_xcd
// then counts workgroups per XCD).
hipError_t launch_decode(int dtype, int head_dim, int gp, bool bins, int block_size,
                         const DecodeParams& p, hipStream_t stream);
// wide: one workgroup per (sequence, q head) (segments with many partials)
// instead of one wave.
hipError_t launch_reduce(int head_dim, int gp, const ReduceParams& p, bool wide,
                         hipStream_t stream);
// Whether the decode launch can take shared-prefix items for this cache dtype,
// head_dim and padded group (split form).
bool prefix_supported(int dtype, int head_dim, int gp);
// Workgroups of the decode kernel one CU can hold at once (occupancy), 0 on error.
int decode_blocks_per_cu(int dtype, int head_dim, int gp, bool bins, int block_size);

// Slots outside [0, num_slots) are skipped.
hipError_t launch_append(const void* k_new, const void* v_new, const int64_t* slots, int batch,
                         void* k_layer, void* v_layer, int kv_heads, int row_bytes,
                         int block_size, int64_t num_slots, hipStream_t stream);
// q8_0 / q4_0 cache (dtype 3 / 4): quantise bf16 new rows
// [batch][kv_heads][head_dim] into the rows at `slots`.
hipError_t launch_append_quant(int dtype, const void* k_new, const void* v_new,
                               const int64_t* slots, int batch, void* k_layer, void* v_layer,
                               int kv_heads, int head_dim, int block_size, int64_t num_slots,
                               hipStream_t stream);
// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned) from mapped
// pinned host memory to device memory with a kernel on `stream`.
hipError_t launch_upload(const void* host_src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_copy_blocks(const int32_t* pairs, int n, void* k_base, void* v_base,
                              int layers, int64_t layer_bytes, int64_t block_bytes,
                              hipStream_t stream);

// Static scratch array (one per device, held until the process ends) for the
// allocation-free decode: its size, and its device address on device `dev`
// (looked up once per device with that device current).
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_address(int dev, void** out);

// Bandwidth probes (pkv_probes.hip). Gather: every K and V tile of one layer
// the uploaded table names, 16 tokens of one kv head each; tile bytes 1024,
// 2048 or 4096 (2-byte caches), blocks of 16 tokens.
struct GatherParams {
  const char* k;               // layer base of K
  const char* v;               // layer base of V
  const int32_t* bt;           // block table [batch][bt_stride]
  const int32_t* cum;          // tiles' prefix sums over the sequences [batch + 1]
  unsigned* out;               // [nwaves * 64] XOR of what each lane read
  int64_t blk_stride;          // bytes per block of one layer (kv_heads tiles)
  int32_t tile;                // bytes per (block, kv head) tile
  int32_t bt_stride;
  int32_t batch;
  int32_t kv_heads;
  int32_t nwaves;
};
hipError_t launch_probe_stream(const void* buf, int64_t bytes, int nwaves, unsigned* out,
                               hipStream_t stream);
hipError_t launch_probe_gather(const GatherParams& p, hipStream_t stream);

#ifdef PKV_TIMELINE
hipError_t copy_timeline(void* dst, size_t bytes);
#endif

}  // namespace pkv
