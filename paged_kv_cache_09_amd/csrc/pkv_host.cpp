// Host side of libpkv: pool descriptor, block manager (free list, reference
// counts, copy-on-write planning), uploads through pinned staging, decode
// scheduling, argument checks and kernel launches. See include/pkv.h for the
// contract of every entry point.
#include "pkv.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <list>
#include <map>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool quantised(int dtype) { return dtype == PKV_Q8_0 || dtype == PKV_Q4_0; }

// Bytes of one stored element (a q8_0 code is one byte; its scales are extra;
// q4_0 is counted by code_row_bytes, two codes per byte). 0: unknown dtype.
int elem_bytes(int dtype) {
  return dtype == PKV_F32 ? 4 : (dtype == PKV_F16 || dtype == PKV_BF16) ? 2
                                : quantised(dtype) ? 1 : 0;
}

// Bytes of one stored row of head_dim elements (codes only when quantised).
int64_t code_row_bytes(int dtype, int head_dim) {
  return dtype == PKV_Q4_0 ? head_dim / 2 : (int64_t)head_dim * elem_bytes(dtype);
}

// Bytes of one (block, kv head) tile of K or V: block_size rows, plus for a
// quantised cache one fp16 scale per 32 elements of each row.
int64_t tile_bytes_of(const pkv_shape* sh) {
  const int64_t codes = (int64_t)sh->block_size * code_row_bytes(sh->dtype, sh->head_dim);
  return quantised(sh->dtype) ? codes + (int64_t)sh->block_size * (sh->head_dim / 32) * 2
                              : codes;
}

// Shape checks shared by pkv_pool_bytes and pkv_kv_pool_alloc.
int check_shape(const pkv_shape* sh) {
  if (!sh) return fail(PKV_EINVAL, "shape is NULL");
  if (sh->layers < 1 || sh->num_blocks < 1 || sh->kv_heads < 1 || sh->max_seqs < 1 ||
      sh->max_seq_len < 1)
    return fail(PKV_EINVAL, "layers, num_blocks, kv_heads, max_seqs and max_seq_len must be >= 1");
  if (elem_bytes(sh->dtype) == 0) return fail(PKV_EINVAL, "unknown dtype %d", sh->dtype);
  if (sh->block_size != 8 && sh->block_size != 16 && sh->block_size != 32)
    return fail(PKV_EUNSUPPORTED, "block_size %d is not supported (8, 16 or 32)", sh->block_size);
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", sh->head_dim);
  if ((int64_t)sh->num_blocks * sh->block_size > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "num_blocks * block_size must fit in int32");
  if (sh->max_seq_len >= (1 << 30))
    return fail(PKV_EUNSUPPORTED, "max_seq_len must be below 2^30");
  return PKV_OK;
}

struct Staging {
  char* host = nullptr;  // coherent pinned host memory
  char* dev = nullptr;   // the same memory as the device addresses it
  size_t bytes = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

}  // namespace

struct pkv_pool {
  pkv_shape shape{};
  bool device = false;
  void* scratch = nullptr;  // this device's static scratch array (allocation-free decode)
  int dev_id = 0;
  int num_cus = 0;
  char* k_base = nullptr;
  char* v_base = nullptr;
  int64_t row_bytes = 0;    // bytes of one stored row (codes only when quantised)
  int64_t tile_bytes = 0;   // 16 rows (+ scales for q8_0)
  int64_t block_bytes = 0;  // kv_heads tiles: one block of one layer, K or V
  int64_t layer_bytes = 0;  // num_blocks blocks
  int32_t max_blocks_per_seq = 0;

  // block manager
  std::vector<int32_t> free_list;  // stack of free ids
  std::vector<int32_t> free_pos;   // index of an id in free_list, -1 when allocated
  std::vector<int32_t> refcount;

  // prefix cache: full blocks registered under a chained hash of the token
  // content from the sequence start. A cached block whose last reference is
  // released stays reusable (evictable, least recently used first) instead of
  // returning to the free list; allocation evicts only when the free list is
  // empty.
  std::unordered_multimap<uint64_t, int32_t> by_hash;
  std::vector<char> cached;
  std::vector<uint64_t> blk_hash;   // lookup key: chained hash of the prefix
  // exact identity of a cached block's prefix: the cached block before it
  // (-1 for a first block) and that block's cache generation when this one
  // was registered (a block id reused for other content gets a new one)
  std::vector<int32_t> blk_parent;
  std::vector<uint32_t> blk_parent_gen, blk_gen;
  std::vector<int32_t> blk_tokens;  // block_size token ids per cached block
  std::list<int32_t> lru;           // evictable blocks, oldest first
  std::vector<std::list<int32_t>::iterator> lru_pos;
  std::vector<char> in_lru;
  int64_t prefix_hits = 0, prefix_evictions = 0;

  // device metadata (library owned). One buffer so that an upload is one copy:
  // [slots int64 max_seqs | ctx int32 max_seqs | cum int32 max_seqs+1 | pad |
  //  table int32 batch x width | pad | decode schedule (up to sched_cap ints)]
  // The schedule follows the table of the current upload (offset off_sched).
  char* d_meta = nullptr;
  size_t off_ctx = 0, off_cum = 0, off_bt = 0, meta_bytes = 0, off_sched = 0;
  int32_t* d_bt = nullptr;
  int32_t* d_ctx = nullptr;
  int32_t* d_cum = nullptr;
  int64_t* d_slots = nullptr;
  std::vector<char> h_stage;  // packed image of one upload
  size_t sched_cap = 0;       // ints the schedule region after the table holds
  int32_t* d_sched = nullptr;  // where the current schedule lives
  int32_t* d_sched_over = nullptr;  // larger schedules (small fixed partitions)
  size_t over_cap = 0;              // ints
  int32_t* d_pairs = nullptr;
  int32_t pairs_cap = 0;  // pairs

  // last upload (host copies)
  bool uploaded = false;
  bool has_slots = false;
  int up_batch = 0;
  int up_stride = 0;
  uint64_t up_gen = 0;
  std::vector<int32_t> h_ctx;
  std::vector<int32_t> h_slotflag;  // per sequence: 1 << 30 when its uploaded slot is >= 0
  std::vector<int32_t> h_cum;
  std::vector<int32_t> h_bt;  // uploaded table (for per-wave descriptors)

  // decode schedule built for (up_gen, partition, gp)
  uint64_t sched_gen = 0;
  int sched_part = -1;
  int sched_gp = 0;
  int sched_nwaves = 0;
  bool sched_needs_merge = false;   // some segment spans several waves
  int sched_max_parts = 0;          // most partials one segment's merge reads
  bool sched_bins = false;          // eight-wave bins form (merges in LDS)
  // shared-prefix groups of the split form: h_sched continues with
  // seqinfo[4 * batch] | items[kItemInts * nitems] | groups[kGroupInts * ngroups]
  int sched_nitems = 0;
  int sched_ngroups = 0;
  int sched_seg_stride = 1;         // partial slots per segment (1 + most chunks)
  int sched_gp_building = 1;        // padded group of the schedule being built
  std::vector<int32_t> h_sched;     // wdesc[8 * nwaves] | seg_w0[nseg] | seg_w1[nseg]
  // The bins schedule, for updating it while lengths only grow: its batch,
  // bin count and group, and per segment (g * batch + s) its tile count and
  // the wave holding its last tile, per wave its tile count, as of the last
  // layout of their bin.
  bool bins_valid = false;
  int bins_batch = 0, bins_nbins = 0, bins_gp = 0;
  double bins_imb0 = 1.0;  // imbalance when the bins were packed
  int64_t n_full_builds = 0, n_updates = 0;
  std::vector<int32_t> bins_seg_tiles, bins_end_wave, bins_count0;
  std::vector<int32_t> bins_li0;  // per bin, its first bin list entry (then the total)

  Staging ring[4];
  int ring_next = 0;
};

namespace {

void uncache(pkv_pool* p, int32_t id) {
  if (!p->cached[id]) return;
  auto range = p->by_hash.equal_range(p->blk_hash[id]);
  for (auto it = range.first; it != range.second; ++it)
    if (it->second == id) {
      p->by_hash.erase(it);
      break;
    }
  p->cached[id] = 0;
}

void lru_remove(pkv_pool* p, int32_t id) {
  p->lru.erase(p->lru_pos[id]);
  p->in_lru[id] = 0;
}

// A block whose last reference is gone: cached blocks stay reusable
// (evictable), others return to the free list.
void free_push(pkv_pool* p, int32_t id) {
  if (p->cached[id]) {
    p->lru_pos[id] = p->lru.insert(p->lru.end(), id);
    p->in_lru[id] = 1;
    return;
  }
  p->free_pos[id] = (int32_t)p->free_list.size();
  p->free_list.push_back(id);
}

// Blocks that can be handed out: free ones plus evictable cached ones.
size_t avail(const pkv_pool* p) { return p->free_list.size() + p->lru.size(); }

void free_remove_list(pkv_pool* p, int32_t id);

// Take a specific unreferenced block out of the free list or the evictable set.
void free_remove(pkv_pool* p, int32_t id) {
  if (p->in_lru[id]) {
    lru_remove(p, id);
    uncache(p, id);
    return;
  }
  free_remove_list(p, id);
}

void free_remove_list(pkv_pool* p, int32_t id) {
  const int32_t i = p->free_pos[id];
  const int32_t last = p->free_list.back();
  p->free_list[i] = last;
  p->free_pos[last] = i;
  p->free_list.pop_back();
  p->free_pos[id] = -1;
}

// Next block to hand out (avail(p) > 0): a free one, else the least recently
// used evictable cached block, whose cache entry is dropped.
int32_t free_pop(pkv_pool* p) {
  if (p->free_list.empty()) {
    const int32_t id = p->lru.front();
    lru_remove(p, id);
    uncache(p, id);
    ++p->prefix_evictions;
    return id;
  }
  const int32_t id = p->free_list.back();
  p->free_list.pop_back();
  p->free_pos[id] = -1;
  return id;
}

size_t round16(size_t n) { return (n + 15) & ~(size_t)15; }

// Copy `bytes` from `src` into the next pinned staging buffer and enqueue its
// copy to `dst` (16-byte aligned, room for round16(bytes)) as a kernel on
// `stream`: the kernel reads the coherent pinned memory over PCIe, which
// avoids a hand-off to a copy engine and back for these small images. The
// buffer is reused only after the kernel that last read it has finished.
// no_alloc: fail instead of growing a staging buffer or creating its event.
int stage_copy(pkv_pool* p, void* dst, const void* src, size_t bytes, hipStream_t stream,
               bool no_alloc = false) {
  const size_t padded = round16(bytes);
  if (no_alloc) {
    const Staging& nx = p->ring[p->ring_next];
    if (nx.bytes < padded || !nx.ev)
      return fail(PKV_EINVAL, "the allocation-free call would need a larger staging buffer "
                              "(%zu bytes)", padded);
  }
  Staging& st = p->ring[p->ring_next];
  p->ring_next = (p->ring_next + 1) % 4;
  hipError_t e;
  if (st.pending) {
    if ((e = hipEventSynchronize(st.ev)) != hipSuccess) return hip_fail(e, "staging wait");
    st.pending = false;
  }
  if (st.bytes < padded) {
    if (st.host) (void)hipHostFree(st.host);
    st.host = st.dev = nullptr;
    st.bytes = 0;
    size_t want = std::max(padded, (size_t)1 << 16);
    if ((e = hipHostMalloc((void**)&st.host, want, hipHostMallocCoherent | hipHostMallocMapped)) !=
        hipSuccess)
      return hip_fail(e, "pinned staging allocation");
    if ((e = hipHostGetDevicePointer((void**)&st.dev, st.host, 0)) != hipSuccess) {
      (void)hipHostFree(st.host);
      st.host = nullptr;
      return hip_fail(e, "pinned staging device address");
    }
    st.bytes = want;
  }
  if (!st.ev && (e = hipEventCreateWithFlags(&st.ev, hipEventDisableTiming)) != hipSuccess)
    return hip_fail(e, "event create");
  std::memcpy(st.host, src, bytes);
  if (padded > bytes) std::memset(st.host + bytes, 0, padded - bytes);
  if ((e = pkv::launch_upload(st.dev, dst, padded, stream)) != hipSuccess)
    return hip_fail(e, "upload launch");
  if ((e = hipEventRecord(st.ev, stream)) != hipSuccess) return hip_fail(e, "event record");
  st.pending = true;
  return PKV_OK;
}

int need_device(const pkv_pool* p) {
  if (!p) return fail(PKV_EINVAL, "pool is NULL");
  if (!p->device) return fail(PKV_EINVAL, "host-only pool (created without device memory)");
  return PKV_OK;
}

// 16-token decode tiles of a sequence (the unit of decode work whatever the block size).
int64_t nblk(int32_t tokens) { return (tokens + pkv::kTile - 1) / pkv::kTile; }
// Block-table entries (blocks) a sequence of `tokens` tokens needs.
int64_t nent(const pkv_pool* p, int64_t tokens) {
  return (tokens + p->shape.block_size - 1) / p->shape.block_size;
}

// Cost, in tiles, of starting a segment inside a wave (balanced schedule).
#ifndef PKV_SEG_START_COST
#define PKV_SEG_START_COST 4
#endif
constexpr int64_t kSegStartCost = PKV_SEG_START_COST;

// Shared-prefix groups (split form; 2-byte caches, head_dim 128, padded GQA
// group <= 4). Sequences whose first tile names the same block(s) are taken in
// batch order, in runs of up to kMaxMembers / gp; a run's shared tiles are the
// leading tiles that name the same blocks in every member and hold only cached
// rows in every member (16 (j + 1) <= ctx - 1: the newest row stays private),
// at most kMaxChunks chunks of at most kChunkTiles tiles. A run of one
// sequence, or sharing fewer than kMinSharedTiles tiles, is not a group.
#ifndef PKV_PREFIX_GROUPS
#define PKV_PREFIX_GROUPS 1
#endif
constexpr bool kPrefixGroups = PKV_PREFIX_GROUPS;
constexpr int kMinSharedTiles = 4;
#ifndef PKV_PREFIX_CHUNK
#define PKV_PREFIX_CHUNK 16
#endif
constexpr int kPrefixChunk = PKV_PREFIX_CHUNK;   // preferred tiles per work item
constexpr int kChunkTiles = 32;    // at most (the chunk's table entries fit one per lane)
constexpr int kMaxChunks = 16;

size_t prefix_sched_ints(const pkv_shape* sh) {
  if (!pkv::prefix_supported(sh->dtype, sh->head_dim, 4)) return 0;
  const size_t half = ((size_t)sh->max_seqs + 1) / 2;  // at most this many groups
  return 4 * (size_t)sh->max_seqs + half * pkv::kGroupInts +
         half * sh->kv_heads * kMaxChunks * pkv::kItemInts;
}

// Whether sequences s and t read tile j from the same block(s).
bool same_tile(const pkv_pool* p, int s, int t, int64_t j) {
  const int32_t* a = p->h_bt.data() + (size_t)s * p->up_stride;
  const int32_t* b = p->h_bt.data() + (size_t)t * p->up_stride;
  switch (p->shape.block_size) {
    case 16: return a[j] == b[j];
    case 32: return a[j >> 1] == b[j >> 1];
    default: return a[2 * j] == b[2 * j] && a[2 * j + 1] == b[2 * j + 1];
  }
}

struct PrefixGroups {
  std::vector<int32_t> pstart;  // per sequence: first private tile
  std::vector<int32_t> nch;     // per sequence: chunks of its group (0: none)
  std::vector<int32_t> items, recs;
  int maxch = 0;
};

void find_groups(const pkv_pool* p, int gp, PrefixGroups& pg) {
  const int B = p->up_batch, H = p->shape.kv_heads;
  pg.pstart.assign(B, 0);
  pg.nch.assign(B, 0);
  const int nm = pkv::kMaxMembers / gp;
  // sequences by the block(s) of their first tile, in batch order
  std::map<int64_t, std::vector<int>> by_first;
  for (int s = 0; s < B; ++s) {
    if ((p->h_ctx[s] - 1) / pkv::kTile < kMinSharedTiles) continue;
    const int32_t* row = p->h_bt.data() + (size_t)s * p->up_stride;
    const int64_t key = p->shape.block_size == 8 ? ((int64_t)row[0] << 32) | (uint32_t)row[1]
                                                 : (int64_t)row[0];
    by_first[key].push_back(s);
  }
  for (auto& kv : by_first) {
    const std::vector<int>& v = kv.second;
    for (size_t a = 0; a + 1 < v.size(); a += nm) {
      const int count = (int)std::min<size_t>(nm, v.size() - a);
      if (count < 2) break;
      int64_t P = (int64_t)kMaxChunks * kChunkTiles;
      for (int k = 0; k < count; ++k) P = std::min<int64_t>(P, (p->h_ctx[v[a + k]] - 1) / pkv::kTile);
      int64_t j = 0;
      for (; j < P; ++j) {
        bool same = true;
        for (int k = 1; k < count && same; ++k) same = same_tile(p, v[a], v[a + k], j);
        if (!same) break;
      }
      P = j;
      if (P < kMinSharedTiles) continue;
      const int nch = (int)std::min<int64_t>(kMaxChunks, (P + kPrefixChunk - 1) / kPrefixChunk);
      const int grp = (int)(pg.recs.size() / pkv::kGroupInts);
      pg.recs.resize(pg.recs.size() + pkv::kGroupInts, 0);
      int32_t* r = pg.recs.data() + (size_t)grp * pkv::kGroupInts;
      r[0] = count;
      r[1] = v[a];
      r[2] = nch;
      for (int k = 0; k < count; ++k) {
        r[3 + k] = v[a + k];
        pg.pstart[v[a + k]] = (int32_t)P;
        pg.nch[v[a + k]] = nch;
      }
      for (int g = 0; g < H; ++g)
        for (int c = 0; c < nch; ++c) {
          const int32_t it[pkv::kItemInts] = {grp, g, (int32_t)(c * P / nch),
                                              (int32_t)((c + 1) * P / nch), c, 0, 0, 0};
          pg.items.insert(pg.items.end(), it, it + pkv::kItemInts);
        }
      pg.maxch = std::max(pg.maxch, nch);
    }
  }
}

// Block id holding tile j's rows 0..7 (or all of them), and for 8-token
// blocks the id holding rows 8..15 (any block when the context ends before).
void tile_blocks(const pkv_pool* p, int s, int64_t j, int32_t& first, int32_t& second) {
  const int32_t* row = p->h_bt.data() + (size_t)s * p->up_stride;
  first = row[j * pkv::kTile / p->shape.block_size];
  second = 0;
  if (p->shape.block_size == 8) second = 16 * j + 8 < p->h_ctx[s] ? row[2 * j + 1] : first;
}

// Build the decode schedule for the current upload.
//   part > 0: one wave per (kv head, sequence, part/16-block partition).
//   part == 0: `target` waves, each an equal share of all tiles.
// Tiles are numbered kv-head-major: x = g * tseq + cum[s] + j.
// h_sched = wdesc[8 * nwaves] | seg_w0[nseg] | seg_w1[nseg]; a wave's
// descriptor holds its first and end tile, the sequence, kv head and block
// index of its first tile, that sequence's length and the first block's id.
bool build_bins(pkv_pool* p, int nbins);
bool update_bins(pkv_pool* p, int nbins);

void build_schedule(pkv_pool* p, int part, int target) {
  p->sched_nitems = 0;
  p->sched_ngroups = 0;
  p->sched_seg_stride = 1;
  PrefixGroups pg;
  if (kPrefixGroups &&
      pkv::prefix_supported(p->shape.dtype, p->shape.head_dim, p->sched_gp_building))
    find_groups(p, p->sched_gp_building, pg);
#ifndef PKV_ITEMS_BY_HEAD
#define PKV_ITEMS_BY_HEAD 1
#endif
  if (PKV_ITEMS_BY_HEAD && !pg.items.empty()) {
    // items ordered by kv head (then group, chunk): the decode launch gives
    // each XCD a contiguous share of them, so a head's prompt tiles are
    // fetched into few L2s
    const size_t n = pg.items.size() / pkv::kItemInts;
    std::vector<int> ord(n);
    for (size_t i = 0; i < n; ++i) ord[i] = (int)i;
    std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) {
      return pg.items[(size_t)a * pkv::kItemInts + 1] < pg.items[(size_t)b * pkv::kItemInts + 1];
    });
    std::vector<int32_t> sorted(pg.items.size());
    for (size_t i = 0; i < n; ++i)
      std::copy_n(pg.items.begin() + (size_t)ord[i] * pkv::kItemInts, pkv::kItemInts,
                  sorted.begin() + i * pkv::kItemInts);
    pg.items.swap(sorted);
  }
  const bool groups = !pg.recs.empty();
  // the eight-wave form: 2-byte and quantised tiles (fp32 tiles spill)
  if (!groups && part == 0 && p->shape.dtype != PKV_F32) {
    const int per_cu = pkv::decode_blocks_per_cu(p->shape.dtype, p->shape.head_dim,
                                                  p->sched_gp_building, true,
                                                  p->shape.block_size);
#ifdef PKV_BINS_PER_CU_MAX
    const int nbins = std::max(1, p->num_cus) * std::min(per_cu, PKV_BINS_PER_CU_MAX);
#else
    const int nbins = std::max(1, p->num_cus) * per_cu;
#endif
    if (per_cu > 0 && update_bins(p, nbins)) {
      ++p->n_updates;
      return;
    }
    ++p->n_full_builds;
    if (per_cu > 0 && build_bins(p, nbins)) return;
  } else {
    ++p->n_full_builds;
  }
  p->bins_valid = false;  // h_sched now holds another form
  const int B = p->up_batch;
  const int H = p->shape.kv_heads;
  if (!groups) {
    pg.pstart.assign(B, 0);
    pg.nch.assign(B, 0);
  }
  // tiles each sequence's own runs cover: from its first private tile on
  std::vector<int64_t> cum(B + 1, 0);
  for (int s = 0; s < B; ++s) cum[s + 1] = cum[s] + nblk(p->h_ctx[s]) - pg.pstart[s];
  const int64_t tseq = cum[B];
  const int64_t T = tseq * H;
  std::vector<int64_t> ws;
  if (part > 0) {
    const int64_t pb = part / pkv::kTile;
    for (int g = 0; g < H; ++g)
      for (int s = 0; s < B; ++s) {
        const int64_t n = nblk(p->h_ctx[s]) - pg.pstart[s];
        for (int64_t j = 0; j < n; j += pb) ws.push_back(g * tseq + cum[s] + j);
      }
  } else {
    // Equal cost per wave, where starting a (kv head, sequence) segment costs
    // kSegStartCost tiles on top of its tiles (q, lengths and the first block
    // id are fetched before the first tile can be requested). Cuts fall where
    // the running cost crosses multiples of total / W.
#ifndef PKV_GROUP_TARGET
#define PKV_GROUP_TARGET 50
#endif
    if (groups) target = (int)((int64_t)target * PKV_GROUP_TARGET / 100);
    const int64_t W = std::max<int64_t>(1, std::min<int64_t>(target, T));
    const int64_t total = T + kSegStartCost * (int64_t)B * H;
    ws.assign(1, 0);
    int64_t cost = 0, x = 0;
    for (int g = 0; g < H && (int64_t)ws.size() < W; ++g)
      for (int s = 0; s < B && (int64_t)ws.size() < W; ++s) {
        cost += kSegStartCost;
        const int64_t n = nblk(p->h_ctx[s]) - pg.pstart[s];
        for (int64_t j = 0; j < n; ++j, ++x) {
          // open a new wave at tile x when the cost before it passes the next cut
          while ((int64_t)ws.size() < W && cost * W >= (int64_t)ws.size() * total && x > ws.back())
            ws.push_back(x);
          ++cost;
        }
      }
  }
  const int W = (int)ws.size();
  ws.push_back(T);
  const int nseg = B * H;
  const size_t nitems = pg.items.size() / pkv::kItemInts;
  const size_t ngroups = pg.recs.size() / pkv::kGroupInts;
  p->h_sched.assign((size_t)8 * W + 2 * (size_t)nseg +
                        (groups ? 4 * (size_t)B + pg.items.size() + pg.recs.size() : 0),
                    0);
  int32_t* desc = p->h_sched.data();
  int32_t* w0 = desc + (size_t)8 * W;
  int32_t* w1 = w0 + nseg;
  // descriptors: walk waves and segments together
  int g = 0, s = 0;
  for (int w = 0; w < W; ++w) {
    const int64_t x0 = ws[w];
    while (g * tseq + cum[s + 1] <= x0) {
      if (++s == B) {
        s = 0;
        ++g;
      }
    }
    const int64_t j0 = x0 - g * tseq - cum[s] + pg.pstart[s];
    int32_t* d = desc + (size_t)8 * w;
    d[0] = (int32_t)x0;
    d[1] = (int32_t)ws[w + 1];
    d[2] = s;
    d[3] = g;
    d[4] = (int32_t)j0;
    d[5] = p->h_ctx[s] | p->h_slotflag[s];
    // the first tile's block(s): rows 8..15 of 8-token blocks in d[7]
    tile_blocks(p, s, j0, d[6], d[7]);
  }
  bool multi = groups;  // grouped sequences always merge their prefix partials
  int max_parts = 0;
  int w = 0;
  for (int gg = 0; gg < H; ++gg)
    for (int ss = 0; ss < B; ++ss) {
      const int seg = gg * B + ss;
      const int64_t first = gg * tseq + cum[ss];
      const int64_t last = first + nblk(p->h_ctx[ss]) - pg.pstart[ss] - 1;
      while (ws[w + 1] <= first) ++w;
      w0[seg] = w;
      int v = w;
      while (ws[v + 1] <= last) ++v;
      w1[seg] = v;
      multi |= v != w;
      max_parts = std::max(max_parts, v - w + 1 + pg.nch[ss]);
    }
  if (groups) {
    int32_t* info = w1 + nseg;
    for (int q = 0; q < B; ++q) {
      info[4 * q] = pg.pstart[q];
      tile_blocks(p, q, pg.pstart[q], info[4 * q + 1], info[4 * q + 2]);
      info[4 * q + 3] = pg.nch[q];
    }
    std::memcpy(info + 4 * (size_t)B, pg.items.data(), pg.items.size() * 4);
    std::memcpy(info + 4 * (size_t)B + pg.items.size(), pg.recs.data(), pg.recs.size() * 4);
    p->sched_nitems = (int)nitems;
    p->sched_ngroups = (int)ngroups;
    p->sched_seg_stride = 1 + pg.maxch;
  }
  p->sched_nwaves = W;
  p->sched_needs_merge = multi;
  p->sched_max_parts = max_parts;
  p->sched_bins = false;
}

int waves_target(const pkv_pool* p, int gp) {
  int per_cu = pkv::decode_blocks_per_cu(p->shape.dtype, p->shape.head_dim, gp, false,
                                         p->shape.block_size);
  per_cu = std::max(1, std::min(per_cu, 32));
  return std::max(1, p->num_cus) * per_cu;
}

// Bins packed no more unevenly than this (max bin / mean bin) are used;
// otherwise the split form with its reduce launch is cheaper. Measured on
// MI355X over 8B-shaped layers of different length mixes, the bins form was
// the faster one up to an imbalance of about 1.39 (bf16), 1.36 (q8_0) and
// 1.26 (q4_0).
constexpr double kBinSlack = 1.25;
// Merges of more partials than this (long contexts at a fixed split) take one
// workgroup per (sequence, q head) instead of one wave.
constexpr int kWideReduce = 64;
using pkv::kBinWaves;

// Bins form of the balanced schedule: whole (kv head, sequence) segments are
// packed into nbins bins, longest processing time first (each segment to the
// least loaded bin of its kv head's XCD group; cost = tiles + kSegStartCost),
// and each bin's tiles are cut into kBinWaves equal-cost runs. Returns false
// (schedule untouched) when
// the packing is too uneven, e.g. a few very long sequences.
//   wdesc per wave: [0] index of its first segment in the bin lists, [1] tile
//   count, [2] sequence, [3] kv head, [4] first block index in that segment,
//   [5] its length (bit 30: has a slot), [6] that block's id, [7] the merges
//   of split segments it takes part in (see below).
//   seglist per listed segment: sequence, kv head, length, first block id.
// Costs of a bin wave's run, per cache type (measured end times of the
// waves of a bin agree with these):
//   skew: waves 0-3 and 4-7 share the four SIMDs, and the older wave of each
//     pair wins issue arbitration, so the older wave's run is longer by skew
//     percent of the mean: a little for the 2-byte caches, whose loop waits
//     on memory, more for the quantised ones, whose loop keeps the SIMD busy;
//   sw: a segment switch inside a run, in tiles;
//   app: the fused append of the new row at the end of a segment, in tiles
//     (quantising the row costs the quantised caches more).
#ifndef PKV_RUN_COSTS_2B
#define PKV_RUN_COSTS_2B 8, 4, 0
#endif
#ifndef PKV_RUN_COSTS_Q8
#define PKV_RUN_COSTS_Q8 30, 8, 1
#endif
#ifndef PKV_RUN_COSTS_Q4
#define PKV_RUN_COSTS_Q4 30, 8, 2
#endif
struct RunCosts {
  double skew, sw, app;
};
RunCosts run_costs(int dtype) {
  if (dtype == PKV_Q4_0) return RunCosts{PKV_RUN_COSTS_Q4};
  if (dtype == PKV_Q8_0) return RunCosts{PKV_RUN_COSTS_Q8};
  return RunCosts{PKV_RUN_COSTS_2B};
}
double slot_capacity(int v, const RunCosts& rc) {
  return v < kBinWaves / 2 ? 1.0 + rc.skew / 200.0 : 1.0 - rc.skew / 200.0;
}

// Cut a bin's segments (tile counts n[i], in order) into nruns contiguous
// runs of its tile sequence (run v starts at bin-local tile start[v]; start[nruns]
// = all tiles), minimising the largest run cost over the run's capacity. A run
// costs one per tile, plus rc.sw for each segment that starts inside it (its
// own first segment is free, since every run has one start) and rc.app for
// each segment that ends in it.
void cut_runs(const std::vector<int64_t>& n, int nruns, const RunCosts& rc, int64_t* start) {
  int64_t tiles = 0;
  for (int64_t k : n) tiles += k;
  double capsum = 0;
  for (int v = 0; v < nruns; ++v) capsum += slot_capacity(v, rc);
  auto pack = [&](double M, int64_t* st) {
    int v = 0;
    double c = 0;
    int64_t x = 0;
    st[0] = 0;
    for (int64_t k : n) {
      int64_t left = k;
      bool seg_start = true;
      while (left > 0) {
        const double sw = seg_start && c > 0 ? rc.sw : 0.0;
        const double cap = M * slot_capacity(v, rc) - c - sw;
        // the run that ends the segment also appends its new row
        int64_t room = (int64_t)std::floor(cap + 1e-9);
        if (room >= left) room = (int64_t)std::floor(cap - rc.app + 1e-9) >= left ? left : left - 1;
        if (room <= 0) {
          if (++v == nruns) return false;
          st[v] = x;
          c = 0;
          continue;
        }
        const int64_t take = std::min(left, room);
        c += sw + (double)take + (take == left ? rc.app : 0.0);
        x += take;
        left -= take;
        seg_start = false;
      }
    }
    for (int u = v + 1; u <= nruns; ++u) st[u] = x;
    return true;
  };
  // Bisection on the largest cost per unit of capacity, to a quarter tile
  // (cuts fall on whole tiles), from a bracket a little above the lower bound
  // (widened to the always feasible all-in-one-run bound if need be).
  double lo = std::max(1.0, (double)tiles / capsum) * 0.999;
  double hi = lo * 1.1 + rc.sw + rc.app + 2.0;
  if (!pack(hi, start)) hi = (double)tiles + (rc.sw + rc.app) * (double)n.size() + 1.0;
  for (int it = 0; it < 40 && hi - lo > 0.25; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (pack(mid, start)) hi = mid;
    else lo = mid;
  }
  pack(hi, start);
}

// Lay out bin b, whose segments are the bin list entries li0 .. li1 - 1 (in
// kv head, then sequence order; words 0-1 of each entry set): refresh the
// entries' lengths and first block ids, cut the bin's tiles into kBinWaves
// runs of balanced cost and write the runs' descriptors, the merge words of
// segments split between runs, each segment's end wave and tile count, and
// each run's tile count (the reference of later in-place updates).
void emit_bin(pkv_pool* p, int b, int li0, int li1) {
  const int B = p->up_batch;
  const int nseg = B * p->shape.kv_heads;
  const int W = p->bins_nbins * kBinWaves;
  int32_t* desc = p->h_sched.data();
  int32_t* list = desc + (size_t)8 * W + 2 * (size_t)nseg;
  std::fill(desc + (size_t)8 * b * kBinWaves, desc + (size_t)8 * (b + 1) * kBinWaves, 0);
  std::vector<int64_t> ntiles;
  ntiles.reserve(li1 - li0);
  for (int li = li0; li < li1; ++li) {
    int32_t* e = list + 4 * (size_t)li;
    const int s = e[0];
    e[2] = p->h_ctx[s] | p->h_slotflag[s];
    e[3] = p->h_bt[(size_t)s * p->up_stride];
    ntiles.push_back(nblk(p->h_ctx[s]));
    p->bins_seg_tiles[(size_t)e[1] * B + s] = (int32_t)ntiles.back();
  }
  // cut the bin's tiles into kBinWaves runs of balanced cost
  int64_t start_tile[kBinWaves + 1];
  cut_runs(ntiles, kBinWaves, run_costs(p->shape.dtype), start_tile);
  // descriptors: walk segments and waves together
  int seg_i = 0;       // index into the bin's entries
  int64_t seg_x0 = 0;  // bin-local tile index where entry seg_i starts
  for (int wv = 0; wv < kBinWaves; ++wv) {
    int32_t* d = desc + (size_t)8 * (b * kBinWaves + wv);
    const int64_t x0 = start_tile[wv], x1 = std::max(start_tile[wv], start_tile[wv + 1]);
    d[1] = (int32_t)(x1 - x0);
    p->bins_count0[b * kBinWaves + wv] = d[1];
    if (x1 <= x0) {
      d[0] = li0;
      continue;
    }
    while (seg_x0 + ntiles[seg_i] <= x0) seg_x0 += ntiles[seg_i++];
    const int32_t* e = list + 4 * (size_t)(li0 + seg_i);
    const int s = e[0];
    const int64_t j0 = x0 - seg_x0;
    d[0] = li0 + seg_i;
    d[2] = s;
    d[3] = e[1];
    d[4] = (int32_t)j0;
    d[5] = p->h_ctx[s] | p->h_slotflag[s];
    d[6] = p->h_bt[(size_t)s * p->up_stride + j0 * pkv::kTile / p->shape.block_size];
  }
  // Segments split between waves: their pieces go to consecutive LDS piece
  // slots (base .. base + n - 1, in holder order), and every holder merges
  // some of the heads (head h goes to holder h mod n). Word 7 of a wave:
  //   bits 0-3  slot of its first segment's piece (when that is split),
  //   bits 4-7  slot of its last segment's piece (split, not its first),
  //   bit 8     it merges heads of its first segment: bits 9-12 base slot,
  //             bits 13-16 holders n, bits 17-19 its index among them;
  //   bit 20    it merges heads of its last segment (index 0): bits 21-24 n.
  int64_t sx = 0;
  int base = 0;
  for (int k = 0; k < li1 - li0; ++k) {
    const int64_t a = sx, e = sx + ntiles[k];  // the segment's bin-local tiles [a, e)
    sx = e;
    int wf = -1, wlast = -1;
    for (int wv = 0; wv < kBinWaves; ++wv) {
      const int64_t x0 = start_tile[wv], x1 = std::max(start_tile[wv], start_tile[wv + 1]);
      if (x1 > x0 && x0 < e && x1 > a) {
        if (wf < 0) wf = wv;
        wlast = wv;
      }
    }
    const int32_t* le = list + 4 * (size_t)(li0 + k);
    if (wlast >= 0) p->bins_end_wave[(size_t)le[1] * B + le[0]] = b * kBinWaves + wlast;
    if (wf < 0 || wlast == wf) continue;
    const int n = wlast - wf + 1;
    for (int wv = wf; wv <= wlast; ++wv) {
      int32_t* d = desc + (size_t)8 * (b * kBinWaves + wv);
      const int slot = base + (wv - wf);
      if (wv == wf && start_tile[wf] < a) {
        // the segment starts inside this wave's run: its last segment
        d[7] |= (slot << 4) | (1 << 20) | (n << 21);
      } else {
        d[7] |= slot | (1 << 8) | (base << 9) | (n << 13) | ((wv - wf) << 17);
      }
    }
    base += n;
  }
}

// Largest bin cost (tiles + kSegStartCost per segment) over the mean.
double bins_imbalance(const pkv_pool* p) {
  const int B = p->up_batch;
  const int nseg = B * p->shape.kv_heads;
  const int32_t* list = p->h_sched.data() + (size_t)8 * p->bins_nbins * kBinWaves + 2 * (size_t)nseg;
  int64_t total = 0, maxload = 0;
  for (int b = 0; b < p->bins_nbins; ++b) {
    int64_t load = 0;
    for (int li = p->bins_li0[b]; li < p->bins_li0[b + 1]; ++li)
      load += nblk(p->h_ctx[list[4 * (size_t)li]]) + kSegStartCost;
    total += load;
    maxload = std::max(maxload, load);
  }
  return total > 0 ? (double)maxload * p->bins_nbins / (double)total : 1.0;
}

bool build_bins(pkv_pool* p, int nbins) {
  const int B = p->up_batch;
  const int H = p->shape.kv_heads;
  const int nseg = B * H;
  p->bins_valid = false;
  if (nbins < 1 || nseg < 1) return false;
  struct Seg {
    int64_t cost;
    int g, s;
  };
  std::vector<Seg> segs;
  segs.reserve(nseg);
  int64_t total = 0;
  for (int g = 0; g < H; ++g)
    for (int s = 0; s < B; ++s) {
      const int64_t c = nblk(p->h_ctx[s]) + kSegStartCost;
      segs.push_back({c, g, s});
      total += c;
    }
  std::stable_sort(segs.begin(), segs.end(),
                   [](const Seg& a, const Seg& b) { return a.cost > b.cost; });
  std::vector<int64_t> load(nbins, 0);
  std::vector<std::vector<int>> members(nbins);
  // XCD affinity: bins [x * nbins / 8, (x + 1) * nbins / 8) run on XCD x. When
  // the kv heads divide evenly among the XCDs, a head's segments go only to
  // its own XCD's bins (group g % ngroups), so tiles that several sequences
  // share (a common prompt) are fetched into one XCD's L2 and re-read there.
  int ngroups = 1;
  if (nbins % pkv::kNumXcd == 0) {
    if (H % pkv::kNumXcd == 0) ngroups = pkv::kNumXcd;
    else if (pkv::kNumXcd % H == 0) ngroups = H;
  }
  const int per_group = nbins / ngroups;
  // per group, a min-heap of (load, bin)
  auto cmp = [](const std::pair<int64_t, int>& a, const std::pair<int64_t, int>& b) {
    return a.first != b.first ? a.first > b.first : a.second > b.second;
  };
  std::vector<std::vector<std::pair<int64_t, int>>> heaps(ngroups);
  for (int gr = 0; gr < ngroups; ++gr) {
    for (int b = gr * per_group; b < (gr + 1) * per_group; ++b) heaps[gr].push_back({0, b});
    std::make_heap(heaps[gr].begin(), heaps[gr].end(), cmp);
  }
  for (int i = 0; i < nseg; ++i) {
    auto& heap = heaps[segs[i].g % ngroups];
    std::pop_heap(heap.begin(), heap.end(), cmp);
    auto top = heap.back();
    heap.pop_back();
    members[top.second].push_back(i);
    load[top.second] += segs[i].cost;
    heap.push_back({load[top.second], top.second});
    std::push_heap(heap.begin(), heap.end(), cmp);
  }
  const int64_t maxload = *std::max_element(load.begin(), load.end());
  if ((double)maxload > kBinSlack * (double)total / nbins) return false;

  const int W = nbins * kBinWaves;
  p->h_sched.assign((size_t)8 * W + 2 * (size_t)nseg + 4 * (size_t)nseg, 0);
  p->bins_nbins = nbins;
  p->bins_end_wave.assign(nseg, 0);
  p->bins_seg_tiles.assign(nseg, 0);
  p->bins_count0.assign(W, 0);
  p->bins_li0.assign(nbins + 1, 0);
  int32_t* list = p->h_sched.data() + (size_t)8 * W + 2 * (size_t)nseg;
  int li = 0;
  for (int b = 0; b < nbins; ++b) {
    std::vector<int>& m = members[b];
    std::sort(m.begin(), m.end(), [&](int a, int c) {
      return segs[a].g != segs[c].g ? segs[a].g < segs[c].g : segs[a].s < segs[c].s;
    });
    p->bins_li0[b] = li;
    for (int i : m) {
      int32_t* e = list + 4 * (size_t)li++;
      e[0] = segs[i].s;
      e[1] = segs[i].g;
    }
    emit_bin(p, b, p->bins_li0[b], li);
  }
  p->bins_li0[nbins] = li;
  p->sched_nwaves = W;
  p->sched_needs_merge = false;
  p->sched_bins = true;
  p->bins_batch = B;
  p->bins_gp = p->sched_gp_building;
  p->bins_imb0 = (double)maxload * nbins / (double)total;
  p->bins_valid = true;
  return true;
}

// A wave may grow by this share of its bin's mean run, rounded down to whole
// tiles, before its bin is cut again (0: the whole schedule is built again
// at every upload). Short runs (a few dozen tiles, where one tile is several
// percent of the launch) take no growth.
#ifndef PKV_BIN_DRIFT
#define PKV_BIN_DRIFT 0.02
#endif
constexpr double kBinDrift = PKV_BIN_DRIFT;
// The bins are packed again once their imbalance (largest over mean) has
// grown this much since they were packed.
constexpr double kBinRepack = 0.01;

// Update the last bins schedule to the current upload, when the batch is the
// same and no (kv head, sequence) segment has fewer tiles than when its bin
// was last laid out (decode steps add one token per sequence): each
// segment's new tiles go to the wave that holds its last tile (the cuts stay
// where they were, so the pieces and merges of split segments are
// unchanged); a bin one of whose waves grew by more than kBinDrift of its
// mean run is cut again; lengths, slot flags and block ids are refreshed.
// Returns false (schedule untouched) when a full build is due: another batch,
// bin count or group, a segment with fewer tiles, or bins whose imbalance has
// grown by kBinRepack since they were packed.
bool update_bins(pkv_pool* p, int nbins) {
  const int B = p->up_batch;
  const int H = p->shape.kv_heads;
  const int nseg = B * H;
  const int W = nbins * kBinWaves;
  if (kBinDrift <= 0 || !p->bins_valid || !p->sched_bins || B != p->bins_batch ||
      nbins != p->bins_nbins || p->sched_gp_building != p->bins_gp ||
      (int)p->bins_count0.size() != W || p->h_sched.size() != (size_t)8 * W + 6 * (size_t)nseg)
    return false;
  std::vector<int32_t> cnt(p->bins_count0);
  for (int g = 0; g < H; ++g)
    for (int s = 0; s < B; ++s) {
      const int64_t d = nblk(p->h_ctx[s]) - p->bins_seg_tiles[(size_t)g * B + s];
      if (d < 0) return false;
      if (d > 0) cnt[p->bins_end_wave[(size_t)g * B + s]] += (int32_t)d;
    }
  if (bins_imbalance(p) > p->bins_imb0 + kBinRepack) return false;
  int32_t* desc = p->h_sched.data();
  int32_t* list = desc + (size_t)8 * W + 2 * (size_t)nseg;
  for (int b = 0; b < nbins; ++b) {
    int64_t sum = 0;
    bool recut = false;
    for (int v = 0; v < kBinWaves; ++v) sum += p->bins_count0[b * kBinWaves + v];
    const int64_t lim = (int64_t)(kBinDrift * (double)sum / kBinWaves);
    for (int v = 0; v < kBinWaves; ++v)
      recut |= cnt[b * kBinWaves + v] - p->bins_count0[b * kBinWaves + v] > lim;
    if (recut) {
      emit_bin(p, b, p->bins_li0[b], p->bins_li0[b + 1]);
      continue;
    }
    for (int v = 0; v < kBinWaves; ++v) {
      const int w = b * kBinWaves + v;
      int32_t* d = desc + (size_t)8 * w;
      d[1] = cnt[w];
      if (cnt[w] == 0) continue;
      const int s = d[2];
      d[5] = p->h_ctx[s] | p->h_slotflag[s];
      d[6] = p->h_bt[(size_t)s * p->up_stride + (size_t)d[4] * pkv::kTile / p->shape.block_size];
    }
    for (int li = p->bins_li0[b]; li < p->bins_li0[b + 1]; ++li) {
      int32_t* e = list + 4 * (size_t)li;
      const int s = e[0];
      e[2] = p->h_ctx[s] | p->h_slotflag[s];
      e[3] = p->h_bt[(size_t)s * p->up_stride];
    }
  }
  return true;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

size_t pkv_pool_bytes(const pkv_shape* sh) {
  if (check_shape(sh) != PKV_OK) return 0;
  return (size_t)sh->layers * sh->num_blocks * 2 * sh->kv_heads * tile_bytes_of(sh);
}

int pkv_kv_pool_alloc(const pkv_shape* sh, void* dev_base, size_t dev_bytes, pkv_pool** out) {
  int rc = check_shape(sh);
  if (rc != PKV_OK) return rc;
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  const int64_t storable = (int64_t)sh->num_blocks * sh->block_size;
  if (sh->max_seq_len > storable)
    return fail(PKV_ECAPACITY,
                "max_seq_len %d exceeds the pool's capacity of %lld tokens "
                "(num_blocks x block_size)",
                sh->max_seq_len, (long long)storable);
  const size_t need = pkv_pool_bytes(sh);
  if (dev_base && dev_bytes < need)
    return fail(PKV_EINVAL, "device buffer holds %zu bytes, the pool needs %zu", dev_bytes, need);
  if (dev_base && (reinterpret_cast<uintptr_t>(dev_base) & 15))
    return fail(PKV_EINVAL, "device buffer must be 16-byte aligned");

  pkv_pool* p = new pkv_pool();
  p->shape = *sh;
  p->row_bytes = code_row_bytes(sh->dtype, sh->head_dim);
  p->tile_bytes = tile_bytes_of(sh);
  p->block_bytes = p->tile_bytes * sh->kv_heads;
  p->layer_bytes = p->block_bytes * sh->num_blocks;
  p->max_blocks_per_seq = (int32_t)((sh->max_seq_len + sh->block_size - 1) / sh->block_size);
  p->refcount.assign(sh->num_blocks, 0);
  p->free_pos.assign(sh->num_blocks, -1);
  p->free_list.reserve(sh->num_blocks);
  p->cached.assign(sh->num_blocks, 0);
  p->in_lru.assign(sh->num_blocks, 0);
  p->lru_pos.resize(sh->num_blocks);
  p->blk_hash.assign(sh->num_blocks, 0);
  p->blk_parent.assign(sh->num_blocks, -1);
  p->blk_parent_gen.assign(sh->num_blocks, 0);
  p->blk_gen.assign(sh->num_blocks, 0);
  for (int32_t id = sh->num_blocks - 1; id >= 0; --id) free_push(p, id);  // pops 0, 1, 2, ...

  if (dev_base) {
    p->device = true;
    p->k_base = static_cast<char*>(dev_base);
    p->v_base = p->k_base + (size_t)sh->layers * p->layer_bytes;
    hipError_t e;
    hipDeviceProp_t prop;
    if ((e = hipGetDevice(&p->dev_id)) != hipSuccess ||
        (e = hipGetDeviceProperties(&prop, p->dev_id)) != hipSuccess) {
      delete p;
      return hip_fail(e, "device query");
    }
    p->num_cus = prop.multiProcessorCount;
    // balanced schedules need 8 ints per wave (at most 32 waves per CU); very
    // small fixed partitions may grow this buffer on first use
    p->sched_cap = (size_t)8 * std::max(p->num_cus, 1) * 32 + 6 * (size_t)sh->max_seqs * sh->kv_heads +
                   prefix_sched_ints(sh);
    p->pairs_cap = sh->max_seqs;
    const size_t bt_bytes = (size_t)sh->max_seqs * p->max_blocks_per_seq * 4;
    p->off_ctx = (size_t)sh->max_seqs * 8;
    p->off_cum = p->off_ctx + (size_t)sh->max_seqs * 4;
    p->off_bt = round16(p->off_cum + ((size_t)sh->max_seqs + 1) * 4);
    p->meta_bytes = round16(p->off_bt + bt_bytes) + round16(p->sched_cap * 4);
    if ((e = hipMalloc((void**)&p->d_meta, p->meta_bytes)) != hipSuccess ||
        (e = hipMalloc((void**)&p->d_pairs, round16((size_t)p->pairs_cap * 8))) != hipSuccess) {
      pkv_kv_pool_free(p);
      return hip_fail(e, "device metadata allocation");
    }
    p->d_slots = reinterpret_cast<int64_t*>(p->d_meta);
    p->d_ctx = reinterpret_cast<int32_t*>(p->d_meta + p->off_ctx);
    p->d_cum = reinterpret_cast<int32_t*>(p->d_meta + p->off_cum);
    p->d_bt = reinterpret_cast<int32_t*>(p->d_meta + p->off_bt);
    // Staging ring sized for the largest image an upload or a schedule can
    // need, with its events: later calls need no allocation for it.
    for (Staging& st : p->ring) {
      const size_t want = std::max(round16(p->meta_bytes), (size_t)1 << 16);
      if ((e = hipHostMalloc((void**)&st.host, want, hipHostMallocCoherent | hipHostMallocMapped)) !=
              hipSuccess ||
          (e = hipHostGetDevicePointer((void**)&st.dev, st.host, 0)) != hipSuccess ||
          (e = hipEventCreateWithFlags(&st.ev, hipEventDisableTiming)) != hipSuccess) {
        pkv_kv_pool_free(p);
        return hip_fail(e, "pinned staging allocation");
      }
      st.bytes = want;
    }
    // the static scratch array of this device (allocation-free decode)
    if ((e = pkv::scratch_address(p->dev_id, &p->scratch)) != hipSuccess) p->scratch = nullptr;
  }
  *out = p;
  return PKV_OK;
}

int pkv_kv_pool_free(pkv_pool* p) {
  if (!p) return PKV_OK;
  if (p->device) (void)hipDeviceSynchronize();
  for (Staging& st : p->ring) {
    if (st.ev) (void)hipEventDestroy(st.ev);
    if (st.host) (void)hipHostFree(st.host);
  }
  (void)hipFree(p->d_meta);
  (void)hipFree(p->d_sched_over);
  (void)hipFree(p->d_pairs);
  delete p;
  return PKV_OK;
}

int pkv_block_alloc(pkv_pool* p, int n, int32_t* ids_out) {
  if (!p || n < 0 || (n > 0 && !ids_out)) return fail(PKV_EINVAL, "bad arguments");
  if ((size_t)n > avail(p))
    return fail(PKV_EOUT_OF_BLOCKS, "asked for %d blocks, %zu free", n, avail(p));
  for (int i = 0; i < n; ++i) {
    const int32_t id = free_pop(p);
    p->refcount[id] = 1;
    ids_out[i] = id;
  }
  return PKV_OK;
}

int pkv_block_claim(pkv_pool* p, const int32_t* ids, int n) {
  if (!p || n < 0 || (n > 0 && !ids)) return fail(PKV_EINVAL, "bad arguments");
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= p->shape.num_blocks)
      return fail(PKV_EINVAL, "block id %d out of range", ids[i]);
    if (p->refcount[ids[i]] != 0) return fail(PKV_EINVAL, "block %d is not free", ids[i]);
  }
  std::vector<int32_t> sorted(ids, ids + n);
  std::sort(sorted.begin(), sorted.end());
  auto dup = std::adjacent_find(sorted.begin(), sorted.end());
  if (dup != sorted.end()) return fail(PKV_EINVAL, "block %d listed twice", *dup);
  for (int i = 0; i < n; ++i) {
    free_remove(p, ids[i]);
    p->refcount[ids[i]] = 1;
  }
  return PKV_OK;
}

int pkv_block_ref(pkv_pool* p, const int32_t* ids, int n) {
  if (!p || n < 0 || (n > 0 && !ids)) return fail(PKV_EINVAL, "bad arguments");
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= p->shape.num_blocks)
      return fail(PKV_EINVAL, "block id %d out of range", ids[i]);
    if (p->refcount[ids[i]] <= 0) return fail(PKV_EINVAL, "block %d is not allocated", ids[i]);
  }
  for (int i = 0; i < n; ++i) ++p->refcount[ids[i]];
  return PKV_OK;
}

int pkv_block_free(pkv_pool* p, const int32_t* ids, int n) {
  if (!p || n < 0 || (n > 0 && !ids)) return fail(PKV_EINVAL, "bad arguments");
  // all-or-nothing: count how many references each listed block loses
  std::vector<std::pair<int32_t, int>> drops;
  drops.reserve(n);
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= p->shape.num_blocks)
      return fail(PKV_EINVAL, "block id %d out of range", ids[i]);
    drops.push_back({ids[i], 1});
  }
  std::sort(drops.begin(), drops.end());
  for (size_t i = 0; i < drops.size();) {
    size_t k = i;
    int cnt = 0;
    while (k < drops.size() && drops[k].first == drops[i].first) cnt += drops[k++].second;
    if (p->refcount[drops[i].first] < cnt)
      return fail(PKV_EINVAL, "block %d has %d references, %d released", drops[i].first,
                  p->refcount[drops[i].first], cnt);
    i = k;
  }
  for (int i = 0; i < n; ++i)
    if (--p->refcount[ids[i]] == 0) free_push(p, ids[i]);
  return PKV_OK;
}

int pkv_block_refcount(const pkv_pool* p, int32_t id) {
  if (!p || id < 0 || id >= p->shape.num_blocks) return fail(PKV_EINVAL, "bad block id");
  return p->refcount[id];
}

namespace {

// Slot assignment for n_new[s] consecutive tokens of each sequence s at
// logical positions ctx_before[s] .. ctx_before[s] + n_new[s] - 1, in batch
// order. Each block index the tokens touch is taken on demand when absent,
// copied first when shared (refcount > 1), else written in place
// (thienlv.com, "PagedAttention là gì?", "How does PagedAttention work?";
// ahmedhaies.com, "PagedAttention: why LLM serving wastes most GPU memory",
// copy-on-write paragraph). All-or-nothing: every check and the block count
// come first, so a failing call changes nothing (a taken block may evict a
// cached one, which could not be undone).
int prepare_core(pkv_pool* p, int32_t* bt, int batch, int max_blocks, const int32_t* ctx_before,
                 const int32_t* n_new, int64_t* slot_out, int64_t slot_capacity,
                 int32_t* cow_out, int cow_capacity, int* n_cow) {
  const int BS = p->shape.block_size;
  struct Undo {
    int64_t entry;
    int32_t old;
  };
  std::vector<Undo> undo;
  std::vector<int32_t> taken, unref;
  int ncow = 0;
  int64_t nslot = 0;
  auto rollback = [&]() {
    for (auto it = undo.rbegin(); it != undo.rend(); ++it) bt[it->entry] = it->old;
    for (int32_t id : taken) {
      p->refcount[id] = 0;
      free_push(p, id);
    }
    for (int32_t id : unref) ++p->refcount[id];
  };
  // Check everything and count the blocks the call takes before changing
  // anything: taking a block may evict a cached one, which a rollback could
  // not restore. The second pass below then cannot fail.
  {
    std::unordered_map<int32_t, int32_t> rc_drop;  // references CoW moves off a block
    int64_t need = 0, nslot_chk = 0;
    int ncow_chk = 0;
    for (int s = 0; s < batch; ++s) {
      const int64_t L0 = ctx_before[s], n = n_new[s], L1 = L0 + n;
      if (L0 < 0 || n < 0 || L1 > p->shape.max_seq_len || (L1 + BS - 1) / BS > max_blocks)
        return fail(PKV_EINVAL, "sequence %d: tokens [%lld, %lld) outside [0, %lld)", s,
                    (long long)L0, (long long)L1,
                    (long long)std::min<int64_t>(p->shape.max_seq_len, (int64_t)max_blocks * BS));
      if (nslot_chk + n > slot_capacity)
        return fail(PKV_EINVAL, "slot buffer too small (%lld)", (long long)slot_capacity);
      nslot_chk += n;
      if (n == 0) continue;
      for (int64_t jb = L0 / BS; jb <= (L1 - 1) / BS; ++jb) {
        const int32_t b = bt[(int64_t)s * max_blocks + jb];
        if (b < 0) {
          ++need;
          continue;
        }
        if (b >= p->shape.num_blocks || p->refcount[b] < 1)
          return fail(PKV_EINVAL, "sequence %d: table entry %d is not an allocated block", s, b);
        auto it = rc_drop.find(b);
        const int32_t rc = p->refcount[b] - (it == rc_drop.end() ? 0 : it->second);
        if (rc > 1) {
          ++need;
          ++ncow_chk;
          ++rc_drop[b];
        }
      }
    }
    if (ncow_chk > 0 && (!cow_out || ncow_chk > cow_capacity))
      return fail(PKV_EINVAL, "copy-on-write pair buffer too small (%d)", cow_capacity);
    if ((size_t)need > avail(p))
      return fail(PKV_EOUT_OF_BLOCKS, "the step needs %lld blocks, %zu free", (long long)need,
                  avail(p));
  }
  for (int s = 0; s < batch; ++s) {
    const int64_t L0 = ctx_before[s], n = n_new[s], L1 = L0 + n;
    if (L0 < 0 || n < 0 || L1 > p->shape.max_seq_len || (L1 + BS - 1) / BS > max_blocks) {
      rollback();
      return fail(PKV_EINVAL, "sequence %d: tokens [%lld, %lld) outside [0, %lld)", s,
                  (long long)L0, (long long)L1,
                  (long long)std::min<int64_t>(p->shape.max_seq_len, (int64_t)max_blocks * BS));
    }
    if (nslot + n > slot_capacity) {
      rollback();
      return fail(PKV_EINVAL, "slot buffer too small (%lld)", (long long)slot_capacity);
    }
    if (n == 0) continue;
    for (int64_t jb = L0 / BS; jb <= (L1 - 1) / BS; ++jb) {
      const int64_t e = (int64_t)s * max_blocks + jb;
      int32_t b = bt[e];
      if (b < 0) {
        if (avail(p) == 0) {
          rollback();
          return fail(PKV_EOUT_OF_BLOCKS, "no free block for sequence %d", s);
        }
        const int32_t nb = free_pop(p);
        p->refcount[nb] = 1;
        taken.push_back(nb);
        undo.push_back({e, b});
        bt[e] = nb;
        b = nb;
      } else {
        if (b >= p->shape.num_blocks || p->refcount[b] < 1) {
          rollback();
          return fail(PKV_EINVAL, "sequence %d: table entry %d is not an allocated block", s, b);
        }
        if (p->refcount[b] == 1 && p->cached[b]) uncache(p, b);  // its content changes
        if (p->refcount[b] > 1) {
          if (!cow_out || ncow >= cow_capacity) {
            rollback();
            return fail(PKV_EINVAL, "copy-on-write pair buffer too small (%d)", cow_capacity);
          }
          if (avail(p) == 0) {
            rollback();
            return fail(PKV_EOUT_OF_BLOCKS, "no free block for copy-on-write of sequence %d", s);
          }
          const int32_t nb = free_pop(p);
          p->refcount[nb] = 1;
          taken.push_back(nb);
          --p->refcount[b];
          unref.push_back(b);
          undo.push_back({e, b});
          cow_out[2 * ncow] = b;
          cow_out[2 * ncow + 1] = nb;
          ++ncow;
          bt[e] = nb;
        }
      }
    }
    for (int64_t pos = L0; pos < L1; ++pos)
      slot_out[nslot++] = (int64_t)bt[(int64_t)s * max_blocks + pos / BS] * BS + pos % BS;
  }
  *n_cow = ncow;
  return PKV_OK;
}

}  // namespace

int pkv_prepare_write(pkv_pool* p, int32_t* bt, int batch, int max_blocks,
                      const int32_t* ctx_before, const int32_t* n_new, int64_t* slot_out,
                      int64_t slot_capacity, int32_t* cow_out, int cow_capacity, int* n_cow) {
  if (!p || !bt || !ctx_before || !n_new || !n_cow || batch < 1 || max_blocks < 1 ||
      slot_capacity < 0 || (slot_capacity > 0 && !slot_out))
    return fail(PKV_EINVAL, "bad arguments");
  if (max_blocks > p->max_blocks_per_seq)
    return fail(PKV_EINVAL, "table width %d exceeds %d blocks (max_seq_len %d)", max_blocks,
                p->max_blocks_per_seq, p->shape.max_seq_len);
  return prepare_core(p, bt, batch, max_blocks, ctx_before, n_new, slot_out, slot_capacity,
                      cow_out, cow_capacity, n_cow);
}

int pkv_prepare_append(pkv_pool* p, int32_t* bt, int batch, int max_blocks,
                       const int32_t* ctx, int64_t* slot_out, int32_t* cow_out,
                       int cow_capacity, int* n_cow) {
  if (!p || !bt || !ctx || !slot_out || !n_cow || batch < 1 || max_blocks < 1)
    return fail(PKV_EINVAL, "bad arguments");
  if (batch > p->shape.max_seqs)
    return fail(PKV_EINVAL, "batch %d exceeds max_seqs %d", batch, p->shape.max_seqs);
  std::vector<int32_t> before(batch), one(batch, 1);
  for (int s = 0; s < batch; ++s) {
    if (ctx[s] < 1 || ctx[s] > p->shape.max_seq_len ||
        nent(p, ctx[s]) > max_blocks)
      return fail(PKV_EINVAL, "sequence %d: context length %d outside [1, %d]", s, ctx[s],
                  std::min<int64_t>(p->shape.max_seq_len,
                                    (int64_t)max_blocks * p->shape.block_size));
    before[s] = ctx[s] - 1;
  }
  return prepare_core(p, bt, batch, max_blocks, before.data(), one.data(), slot_out, batch,
                      cow_out, cow_capacity, n_cow);
}

int pkv_block_table_upload(pkv_pool* p, const int32_t* bt, int batch, int max_blocks,
                           const int32_t* ctx, const int64_t* slots, uintptr_t stream_u) {
  int rc = need_device(p);
  if (rc != PKV_OK) return rc;
  if (!bt || !ctx || batch < 1 || max_blocks < 1) return fail(PKV_EINVAL, "bad arguments");
  if (batch > p->shape.max_seqs)
    return fail(PKV_EINVAL, "batch %d exceeds max_seqs %d", batch, p->shape.max_seqs);
  if (max_blocks > p->max_blocks_per_seq)
    return fail(PKV_EINVAL, "table width %d exceeds %d blocks (max_seq_len %d)", max_blocks,
                p->max_blocks_per_seq, p->shape.max_seq_len);
  std::vector<int32_t> cum(batch + 1);
  cum[0] = 0;
  for (int s = 0; s < batch; ++s) {
    const int32_t L = ctx[s];
    const int BS = p->shape.block_size;
    if (L < 1 || L > p->shape.max_seq_len || nent(p, L) > max_blocks)
      return fail(PKV_EINVAL, "sequence %d: context length %d outside [1, %d]", s, L,
                  std::min<int64_t>(p->shape.max_seq_len, (int64_t)max_blocks * BS));
    const int64_t n = nblk(L);  // tiles
    for (int64_t j = 0; j < nent(p, L); ++j) {
      const int32_t b = bt[(int64_t)s * max_blocks + j];
      if (b < 0 || b >= p->shape.num_blocks)
        return fail(PKV_EINVAL, "sequence %d: block table entry %lld = %d out of range", s,
                    (long long)j, b);
    }
    if ((int64_t)cum[s] + n > INT32_MAX / p->shape.kv_heads)
      return fail(PKV_EUNSUPPORTED, "too many tiles in one batch");
    cum[s + 1] = cum[s] + (int32_t)n;
  }
  if (slots) {
    const int BS = p->shape.block_size;
    const int64_t lim = (int64_t)p->shape.num_blocks * BS;
    std::vector<int64_t> seen;
    seen.reserve(batch);
    for (int s = 0; s < batch; ++s) {
      if (slots[s] >= lim) return fail(PKV_EINVAL, "slot %lld out of range", (long long)slots[s]);
      if (slots[s] >= 0) seen.push_back(slots[s]);
    }
    for (int s = 0; s < batch; ++s) {
      if (slots[s] < 0) continue;
      const int32_t pos = ctx[s] - 1;
      const int64_t want =
          (int64_t)bt[(int64_t)s * max_blocks + pos / BS] * BS + pos % BS;
      if (slots[s] != want)
        return fail(PKV_EINVAL, "sequence %d: slot %lld is not the table position %lld of its "
                    "new token", s, (long long)slots[s], (long long)want);
    }
    std::sort(seen.begin(), seen.end());
    for (size_t i = 1; i < seen.size(); ++i)
      if (seen[i] == seen[i - 1])
        return fail(PKV_EINVAL, "slot %lld appears twice (the appends would race)",
                    (long long)seen[i]);
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_u);
  // host copies first: the decode schedule is built from them
  p->uploaded = false;
  p->has_slots = slots != nullptr;
  p->up_batch = batch;
  p->up_stride = max_blocks;
  p->h_ctx.assign(ctx, ctx + batch);
  // the kernels read the lengths with bit 30 set where the sequence has a slot
  // (its new row is appended by a fused decode)
  p->h_slotflag.assign(batch, 0);
  if (slots)
    for (int s = 0; s < batch; ++s) p->h_slotflag[s] = slots[s] >= 0 ? (1 << 30) : 0;
  p->h_cum = std::move(cum);
  p->h_bt.assign(bt, bt + (size_t)batch * max_blocks);
  ++p->up_gen;
  // Pack slots, lengths, prefix sums, the table and — when a decode has run
  // before — the schedule for that decode's partition setting and group into
  // one image: one copy per step.
  const size_t tbl_end = p->off_bt + (size_t)batch * max_blocks * 4;
  const size_t off_sched = round16(tbl_end);
  size_t bytes = tbl_end;
  bool packed = false;
  if (p->sched_part >= 0) {
    p->sched_gp_building = p->sched_gp;
    build_schedule(p, p->sched_part, waves_target(p, p->sched_gp));
    if (p->h_sched.size() <= p->sched_cap) {
      packed = true;
      bytes = off_sched + p->h_sched.size() * 4;
    }
  }
  p->h_stage.assign(bytes, 0);
  char* img = p->h_stage.data();
  if (slots) std::memcpy(img, slots, (size_t)batch * 8);
  for (int s = 0; s < batch; ++s)
    reinterpret_cast<int32_t*>(img + p->off_ctx)[s] = ctx[s] | p->h_slotflag[s];
  std::memcpy(img + p->off_cum, p->h_cum.data(), (size_t)(batch + 1) * 4);
  std::memcpy(img + p->off_bt, bt, (size_t)batch * max_blocks * 4);
  if (packed) std::memcpy(img + off_sched, p->h_sched.data(), p->h_sched.size() * 4);
  if ((rc = stage_copy(p, p->d_meta, img, bytes, stream))) return rc;
  p->off_sched = off_sched;
  if (packed) {
    p->d_sched = reinterpret_cast<int32_t*>(p->d_meta + off_sched);
    p->sched_gen = p->up_gen;
  }
  p->uploaded = true;
  return PKV_OK;
}

int pkv_copy_blocks(pkv_pool* p, const int32_t* pairs, int n, uintptr_t stream_u) {
  int rc = need_device(p);
  if (rc != PKV_OK) return rc;
  if (n == 0) return PKV_OK;
  if (n < 0 || !pairs) return fail(PKV_EINVAL, "bad arguments");
  if (n > p->pairs_cap) return fail(PKV_EINVAL, "%d pairs exceed capacity %d", n, p->pairs_cap);
  std::vector<int32_t> dsts;
  for (int i = 0; i < n; ++i) {
    for (int k = 0; k < 2; ++k)
      if (pairs[2 * i + k] < 0 || pairs[2 * i + k] >= p->shape.num_blocks)
        return fail(PKV_EINVAL, "pair %d: block id %d out of range", i, pairs[2 * i + k]);
    if (pairs[2 * i] == pairs[2 * i + 1]) return fail(PKV_EINVAL, "pair %d copies onto itself", i);
    dsts.push_back(pairs[2 * i + 1]);
  }
  std::sort(dsts.begin(), dsts.end());
  if (std::adjacent_find(dsts.begin(), dsts.end()) != dsts.end())
    return fail(PKV_EINVAL, "two pairs copy into the same block");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_u);
  if ((rc = stage_copy(p, p->d_pairs, pairs, (size_t)n * 8, stream))) return rc;
  hipError_t e = pkv::launch_copy_blocks(p->d_pairs, n, p->k_base, p->v_base, p->shape.layers,
                                         p->layer_bytes, p->block_bytes, stream);
  if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
  return PKV_OK;
}

int pkv_kv_append(pkv_pool* p, int layer, const void* k_new, const void* v_new,
                  const int64_t* dev_slots, int batch, uintptr_t stream_u) {
  int rc = need_device(p);
  if (rc != PKV_OK) return rc;
  if (layer < 0 || layer >= p->shape.layers) return fail(PKV_EINVAL, "layer %d out of range", layer);
  if (!k_new || !v_new || batch < 1) return fail(PKV_EINVAL, "bad arguments");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  const int64_t* slots = dev_slots;
  if (!slots) {
    if (!p->uploaded || !p->has_slots)
      return fail(PKV_EINVAL, "no slots given and none uploaded");
    if (batch != p->up_batch)
      return fail(PKV_EINVAL, "batch %d differs from the uploaded batch %d", batch, p->up_batch);
    slots = p->d_slots;
  }
  char* kl = p->k_base + (size_t)layer * p->layer_bytes;
  char* vl = p->v_base + (size_t)layer * p->layer_bytes;
  const int64_t num_slots = (int64_t)p->shape.num_blocks * p->shape.block_size;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_u);
  hipError_t e =
      quantised(p->shape.dtype)
          ? pkv::launch_append_quant(p->shape.dtype, k_new, v_new, slots, batch, kl, vl,
                                     p->shape.kv_heads, p->shape.head_dim, p->shape.block_size,
                                     num_slots, stream)
          : pkv::launch_append(k_new, v_new, slots, batch, kl, vl, p->shape.kv_heads,
                               (int)p->row_bytes, p->shape.block_size, num_slots, stream);
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  return PKV_OK;
}

size_t pkv_decode_workspace_bytes(const pkv_pool* p, int batch, int q_heads,
                                  int partition_tokens) {
  if (!p || batch < 1 || q_heads < 1 || q_heads % p->shape.kv_heads) return 0;
  const int group = q_heads / p->shape.kv_heads;
  if (group > pkv::kMaxGroup) return 0;
  const int gp = pkv::padded_group(group);
  const int64_t nseg = (int64_t)batch * p->shape.kv_heads;
  int64_t waves;
  if (partition_tokens > 0) {
    const int64_t pb = std::max(1, partition_tokens / pkv::kTile);
    waves = nseg * ((nblk(p->shape.max_seq_len) + pb - 1) / pb);  // tiles per sequence
  } else {
    waves = std::max<int64_t>(1, std::max(p->num_cus, 1) * 32);
  }
  // shared-prefix partials: up to kMaxChunks slots before each segment's own
  const int64_t stride =
      kPrefixGroups && pkv::prefix_supported(p->shape.dtype, p->shape.head_dim, gp)
          ? 1 + kMaxChunks : 1;
  return (size_t)(nseg * stride + waves) * gp * (p->shape.head_dim + 2) * sizeof(float);
}

namespace {

// no_alloc: the partials live in the device's static scratch array, and a
// call that would allocate (schedule or staging growth) fails instead.
int decode_impl(pkv_pool* p, int layer, const void* k_new, const void* v_new, const void* q,
                int q_heads, float scale, float* out, int partition_tokens, void* ws,
                size_t ws_bytes, uintptr_t stream_u, bool no_alloc = false) {
  int rc = need_device(p);
  if (rc != PKV_OK) return rc;
  if (no_alloc) {
    if (!p->scratch) return fail(PKV_EHIP, "no scratch array on this device");
    ws = p->scratch;
    ws_bytes = pkv::kScratchBytes;
  }
  if (!p->uploaded) return fail(PKV_EINVAL, "no block table uploaded");
  if (layer < 0 || layer >= p->shape.layers) return fail(PKV_EINVAL, "layer %d out of range", layer);
  if (!q || !out) return fail(PKV_EINVAL, "q and out must be device pointers");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(PKV_EINVAL, "q and out must be 16-byte aligned");
  if (k_new) {
    if (!v_new) return fail(PKV_EINVAL, "k_new without v_new");
    if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
      return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
    if (!p->has_slots) return fail(PKV_EINVAL, "append needs slots in the last upload");
  }
  if (q_heads < 1 || q_heads % p->shape.kv_heads)
    return fail(PKV_EINVAL, "q_heads %d is not a multiple of kv_heads %d", q_heads,
                p->shape.kv_heads);
  const int group = q_heads / p->shape.kv_heads;
  if (group > pkv::kMaxGroup)
    return fail(PKV_EUNSUPPORTED, "GQA group %d exceeds %d", group, pkv::kMaxGroup);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale must be finite");
  if (partition_tokens < 0 || partition_tokens % pkv::kTile)
    return fail(PKV_EINVAL, "partition_tokens %d must be 0 or a positive multiple of 16",
                partition_tokens);
  const int gp = pkv::padded_group(group);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_u);
  hipError_t e;

  if (p->sched_gen != p->up_gen || p->sched_part != partition_tokens || p->sched_gp != gp) {
    p->sched_gp_building = gp;
    build_schedule(p, partition_tokens, waves_target(p, gp));
    if (no_alloc && p->sched_needs_merge) {
      // partials beyond the static array: refused before anything is staged
      const int64_t np = (int64_t)p->up_batch * p->shape.kv_heads * p->sched_seg_stride +
                         p->sched_nwaves;
      const size_t nb = (size_t)np * gp * (p->shape.head_dim + 2) * sizeof(float);
      if (nb > pkv::kScratchBytes) {
        p->sched_gen = 0;
        return fail(PKV_EUNSUPPORTED,
                    "the split partials need %zu bytes, more than the static scratch array (%zu)",
                    nb, pkv::kScratchBytes);
      }
    }
    int32_t* dst = reinterpret_cast<int32_t*>(p->d_meta + p->off_sched);
    if (p->h_sched.size() > p->sched_cap) {  // rare: very small fixed partitions
      if (no_alloc && p->h_sched.size() > p->over_cap) {
        p->sched_gen = 0;
        return fail(PKV_EINVAL, "the allocation-free call would need a larger schedule buffer "
                                "(%zu ints; partition %d)", p->h_sched.size(), partition_tokens);
      }
      if (p->h_sched.size() > p->over_cap) {
        if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "sync");
        (void)hipFree(p->d_sched_over);
        p->d_sched_over = nullptr;
        p->over_cap = p->h_sched.size() + p->h_sched.size() / 2;
        if ((e = hipMalloc((void**)&p->d_sched_over, round16(p->over_cap * 4))) != hipSuccess) {
          p->over_cap = 0;
          p->sched_gen = 0;
          return hip_fail(e, "schedule allocation");
        }
      }
      dst = p->d_sched_over;
    }
    if ((rc = stage_copy(p, dst, p->h_sched.data(), p->h_sched.size() * 4, stream, no_alloc))) {
      p->sched_gen = 0;
      return rc;
    }
    p->d_sched = dst;
    p->sched_gen = p->up_gen;
    p->sched_part = partition_tokens;
    p->sched_gp = gp;
  }
  const int B = p->up_batch;
  const int W = p->sched_nwaves;
  const int64_t nseg = (int64_t)B * p->shape.kv_heads;
  const int64_t nparts = nseg * p->sched_seg_stride + W;
  const size_t need = (size_t)nparts * gp * (p->shape.head_dim + 2) * sizeof(float);
  if (p->sched_needs_merge && (ws_bytes < need || !ws))
    return fail(no_alloc ? PKV_EUNSUPPORTED : PKV_EINVAL,
                "%s of %zu bytes is smaller than the %zu needed",
                no_alloc ? "the static scratch array" : "workspace", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 15)
    return fail(PKV_EINVAL, "workspace must be 16-byte aligned");
  float* part = static_cast<float*>(ws);

  pkv::DecodeParams dp{};
  dp.k = p->k_base + (size_t)layer * p->layer_bytes;
  dp.v = p->v_base + (size_t)layer * p->layer_bytes;
  dp.bt = p->d_bt;
  dp.ctx = p->d_ctx;
  dp.wdesc = p->d_sched;
  dp.seg_w0 = p->d_sched + (size_t)8 * W;
  dp.seg_w1 = dp.seg_w0 + nseg;
  dp.seglist = dp.seg_w1 + nseg;
  dp.q = q;
  dp.k_new = k_new;
  dp.v_new = v_new;
  dp.slots = p->d_slots;
  dp.out = out;
  dp.part_o = part;
  dp.part_ml = part + (size_t)nparts * gp * p->shape.head_dim;
  dp.scale_log2 = scale * 1.4426950408889634f;
  dp.bt_stride = p->up_stride;
  dp.batch = B;
  dp.kv_heads = p->shape.kv_heads;
  dp.q_heads = q_heads;
  dp.group = group;
  dp.nwaves = W;
  dp.seg_stride = p->sched_seg_stride;
  dp.seqinfo = p->sched_ngroups > 0 ? dp.seg_w1 + nseg : nullptr;
  if (p->sched_ngroups > 0) {
    // shared-prefix items run in the same launch, ahead of the private runs
    dp.items = dp.seqinfo + 4 * (size_t)B;
    dp.groups = dp.items + (size_t)pkv::kItemInts * p->sched_nitems;
    dp.nitems = p->sched_nitems;
    dp.nprefix = (p->sched_nitems + pkv::kNumXcd - 1) / pkv::kNumXcd * pkv::kNumXcd;
  }
  const int groups = p->sched_bins ? W / kBinWaves : W;  // workgroups: bins, or one per wave
  dp.waves_per_xcd = (groups + pkv::kNumXcd - 1) / pkv::kNumXcd;
  e = pkv::launch_decode(p->shape.dtype, p->shape.head_dim, gp, p->sched_bins,
                         p->shape.block_size, dp, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (p->sched_needs_merge) {
    pkv::ReduceParams rp{};
    rp.part_o = dp.part_o;
    rp.part_ml = dp.part_ml;
    rp.seg_w0 = dp.seg_w0;
    rp.seg_w1 = dp.seg_w1;
    rp.out = out;
    rp.batch = B;
    rp.kv_heads = p->shape.kv_heads;
    rp.q_heads = q_heads;
    rp.group = group;
    rp.seqinfo = dp.seqinfo;
    rp.seg_stride = dp.seg_stride;
    e = pkv::launch_reduce(p->shape.head_dim, gp, rp, p->sched_max_parts > kWideReduce, stream);
    if (e != hipSuccess) return hip_fail(e, "reduce launch");
  }
  return PKV_OK;
}

}  // namespace

int pkv_paged_attn_decode(pkv_pool* p, int layer, const void* q, int q_heads, float scale,
                          float* out, int partition_tokens, void* ws, size_t ws_bytes,
                          uintptr_t stream) {
  return decode_impl(p, layer, nullptr, nullptr, q, q_heads, scale, out, partition_tokens, ws,
                     ws_bytes, stream);
}

int pkv_paged_attn_decode_noalloc(pkv_pool* p, int layer, const void* q, int q_heads,
                                  float scale, float* out, int partition_tokens,
                                  uintptr_t stream) {
  return decode_impl(p, layer, nullptr, nullptr, q, q_heads, scale, out, partition_tokens,
                     nullptr, 0, stream, true);
}

int pkv_append_paged_attn_decode(pkv_pool* p, int layer, const void* k_new, const void* v_new,
                                 const void* q, int q_heads, float scale, float* out,
                                 int partition_tokens, void* ws, size_t ws_bytes,
                                 uintptr_t stream) {
  if (!k_new || !v_new) return fail(PKV_EINVAL, "k_new and v_new are required");
  return decode_impl(p, layer, k_new, v_new, q, q_heads, scale, out, partition_tokens, ws,
                     ws_bytes, stream);
}

}  // extern "C"

namespace {

// FNV-1a, 64-bit (Fowler, Noll, Vo): offset basis 14695981039346656037,
// prime 1099511628211, over the little-endian bytes of the parent block's
// hash followed by the block's token ids.
uint64_t block_hash(uint64_t parent, const int32_t* tokens, int n) {
  uint64_t h = 14695981039346656037ull;
  auto mix = [&h](uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (v >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  mix(parent, 8);
  for (int i = 0; i < n; ++i) mix((uint32_t)tokens[i], 4);
  return h;
}

// The cached block holding `tokens` right after the cached block `parent`
// (-1: at the start of a prompt) whose cache generation is `parent_gen`, or
// -1. The hash only narrows the search; the match is exact.
int32_t cache_find(const pkv_pool* p, uint64_t h, int32_t parent, uint32_t parent_gen,
                   const int32_t* tokens) {
  const int BS = p->shape.block_size;
  auto range = p->by_hash.equal_range(h);
  for (auto it = range.first; it != range.second; ++it) {
    const int32_t id = it->second;
    if (p->blk_parent[id] == parent && (parent < 0 || p->blk_parent_gen[id] == parent_gen) &&
        std::memcmp(&p->blk_tokens[(size_t)id * BS], tokens, (size_t)BS * 4) == 0)
      return id;
  }
  return -1;
}

}  // namespace

extern "C" {

int pkv_prefix_match(pkv_pool* p, const int32_t* tokens, int n_tokens, int32_t* ids_out,
                     int max_ids) {
  if (!p || n_tokens < 0 || (n_tokens > 0 && !tokens) || max_ids < 0 ||
      (max_ids > 0 && !ids_out))
    return fail(PKV_EINVAL, "bad arguments");
  const int BS = p->shape.block_size;
  uint64_t h_prev = 0;
  int32_t parent = -1;
  uint32_t parent_gen = 0;
  int k = 0;
  for (; k < max_ids && (int64_t)(k + 1) * BS <= n_tokens; ++k) {
    const int32_t* t = tokens + (size_t)k * BS;
    const uint64_t h = block_hash(h_prev, t, BS);
    const int32_t id = cache_find(p, h, parent, parent_gen, t);
    if (id < 0) break;
    if (p->refcount[id] == 0) lru_remove(p, id);
    ++p->refcount[id];
    ids_out[k] = id;
    h_prev = h;
    parent = id;
    parent_gen = p->blk_gen[id];
  }
  p->prefix_hits += k;
  return k;
}

int pkv_prefix_insert(pkv_pool* p, const int32_t* tokens, int n_tokens, const int32_t* bt_row,
                      int n_entries) {
  if (!p || n_tokens < 0 || (n_tokens > 0 && (!tokens || !bt_row)) || n_entries < 0)
    return fail(PKV_EINVAL, "bad arguments");
  const int BS = p->shape.block_size;
  const int full = std::min<int64_t>(n_tokens / BS, n_entries);
  for (int j = 0; j < full; ++j) {
    const int32_t id = bt_row[j];
    if (id < 0 || id >= p->shape.num_blocks || p->refcount[id] < 1)
      return fail(PKV_EINVAL, "entry %d = %d is not an allocated block", j, id);
  }
  uint64_t h_prev = 0;
  int32_t parent = -1;
  uint32_t parent_gen = 0;
  int added = 0;
  for (int j = 0; j < full; ++j) {
    const int32_t id = bt_row[j];
    const int32_t* t = tokens + (size_t)j * BS;
    const uint64_t h = block_hash(h_prev, t, BS);
    int32_t canon = cache_find(p, h, parent, parent_gen, t);
    if (canon < 0) {
      // a block cached under another prefix cannot be keyed again: the
      // chain of this prompt stops here
      if (p->cached[id]) break;
      p->cached[id] = 1;
      p->blk_hash[id] = h;
      p->blk_parent[id] = parent;
      p->blk_parent_gen[id] = parent_gen;
      ++p->blk_gen[id];
      if (p->blk_tokens.empty()) p->blk_tokens.assign((size_t)p->shape.num_blocks * BS, 0);
      std::memcpy(&p->blk_tokens[(size_t)id * BS], t, (size_t)BS * 4);
      p->by_hash.emplace(h, id);
      ++added;
      canon = id;
    }
    h_prev = h;
    parent = canon;
    parent_gen = p->blk_gen[canon];
  }
  return added;
}

int pkv_prefix_stats(const pkv_pool* p, int64_t stats[4]) {
  if (!p || !stats) return fail(PKV_EINVAL, "bad arguments");
  int64_t n = 0;
  for (char c : p->cached) n += c;
  stats[0] = n;
  stats[1] = (int64_t)p->lru.size();
  stats[2] = p->prefix_hits;
  stats[3] = p->prefix_evictions;
  return PKV_OK;
}

#ifdef PKV_TIMELINE
int pkv_debug_timeline(void* host_dst, size_t bytes) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = pkv::copy_timeline(host_dst, bytes);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "timeline copy");
}
#endif

int pkv_pool_stats(const pkv_pool* p, int64_t stats[4]) {
  if (!p || !stats) return fail(PKV_EINVAL, "bad arguments");
  int64_t shared = 0;
  for (int32_t r : p->refcount) shared += r > 1;
  int64_t waste = 0;
  for (int32_t L : p->h_ctx) waste += nent(p, L) * p->shape.block_size - L;
  stats[0] = (int64_t)avail(p);
  stats[1] = p->shape.num_blocks - stats[0];
  stats[2] = shared;
  stats[3] = waste;
  return PKV_OK;
}

int pkv_probe_stream_read(const void* dev_buf, int64_t bytes, uint32_t* dev_out, int waves,
                          uintptr_t stream_u) {
  if (!dev_buf || !dev_out || bytes < 16 || (bytes & 15) || waves < 1 || waves > (1 << 20) ||
      (reinterpret_cast<uintptr_t>(dev_buf) & 15))
    return fail(PKV_EINVAL, "bad arguments");
  hipError_t e = pkv::launch_probe_stream(dev_buf, bytes, waves, dev_out,
                                          reinterpret_cast<hipStream_t>(stream_u));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "stream probe launch");
}

int pkv_probe_gather(const pkv_pool* p, int layer, uint32_t* dev_out, int waves,
                     uintptr_t stream_u) {
  int rc = need_device(p);
  if (rc != PKV_OK) return rc;
  if (!dev_out || waves < 1 || waves > (1 << 20) || layer < 0 || layer >= p->shape.layers)
    return fail(PKV_EINVAL, "bad arguments");
  if (!p->uploaded) return fail(PKV_EINVAL, "no block table uploaded");
  if (p->shape.block_size != 16 || (p->tile_bytes != 1024 && p->tile_bytes != 2048 &&
                                    p->tile_bytes != 4096))
    return fail(PKV_EUNSUPPORTED, "the gather probe takes 2-byte caches in blocks of 16");
  pkv::GatherParams g{};
  g.k = p->k_base + (size_t)layer * p->layer_bytes;
  g.v = p->v_base + (size_t)layer * p->layer_bytes;
  g.bt = p->d_bt;
  g.cum = p->d_cum;
  g.out = dev_out;
  g.blk_stride = p->block_bytes;
  g.tile = (int32_t)p->tile_bytes;
  g.bt_stride = p->up_stride;
  g.batch = p->up_batch;
  g.kv_heads = p->shape.kv_heads;
  g.nwaves = waves;
  hipError_t e = pkv::launch_probe_gather(g, reinterpret_cast<hipStream_t>(stream_u));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "gather probe launch");
}

int pkv_schedule_stats(const pkv_pool* p, int64_t stats[4]) {
  if (!p || !stats) return fail(PKV_EINVAL, "bad arguments");
  stats[0] = p->n_full_builds;
  stats[1] = p->n_updates;
  stats[2] = p->sched_bins ? 1 : 0;
  stats[3] = p->sched_nwaves;
  return PKV_OK;
}

}  // extern "C"
