// C ABI of the gfx950 SPICY-KV library: host-side validation, workspace
// carving and launches on the caller's stream.  No allocation and no
// synchronisation; the only state is the per-device address of the
// no-allocation decode's scratch array, looked up once per device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "launch.h"
#include "spicy.h"
#include "spicy_device.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int32_t kMaxKvHeads = 16;
constexpr int32_t kMaxGroup = 16;       // query heads per KV head (MFMA columns)
// Page groups: one workgroup of kWpg wavefronts each; the MFMA kernel's
// register use allows two wavefronts per SIMD, so two such workgroups per CU
// run at a time (kRound on the chip).  Every unit (a tile-set of query rows
// and the pages it reads) is cut into about kTarget / units groups (at least
// one page per wavefront), and the prefix units take what is left of one
// round: a workgroup that starts only when another ends pays the whole
// latency chain of the call again (measured: 5 groups of the 7B layer's
// units, 320 workgroups of 8 wavefronts, 23 us against 16).
constexpr int32_t kWpg = 4;
constexpr int32_t kRound = 512;           // 256 CUs x 2 workgroups
constexpr int32_t kTarget = 192;          // groups per role: about 3/4 of the CUs
constexpr int32_t kF32Chunk = 16;         // fp32 kernel: pages per group (4 wavefronts x 4 pages)
constexpr int32_t kMaxSplits = 256;
constexpr int32_t kMaxGridY = 65535;      // grid y/z extent limit (sequences, heads)
constexpr int32_t kMaxPagesPerSeq = 1 << 23;  // entry ids fit the 27 bits a C-point item keeps

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

spicy_status check_cache(const spicy_cache* c) {
    if (!c) return SPICY_ERR_ARG;
    if (c->dtype != SPICY_F32 && c->dtype != SPICY_BF16) return SPICY_ERR_ARG;
    if (c->num_kv_heads < 1 || c->num_pages < 0) return SPICY_ERR_ARG;
    if (!head_dim_ok(c->head_dim) || c->num_kv_heads > kMaxKvHeads) return SPICY_ERR_UNSUPPORTED;
    if (c->num_pages > 0 && (!c->k || !c->v || !c->ab)) return SPICY_ERR_ARG;
    return SPICY_OK;
}

int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

// Page groups of one decode call: prefix_groups groups of the shared prefix
// (slots 0 .. prefix_groups-1), then priv_groups groups of each (sequence,
// KV head)'s private pages [P, max_pages).
struct DecodePlan {
    int32_t prefix_chunk = 0;
    int32_t prefix_groups = 0;
    int32_t priv_chunk = 0;
    int32_t priv_groups = 0;
    int32_t wpg = kWpg;
    int32_t slots() const { return prefix_groups + priv_groups; }
};

// 16-row query tiles of one (sequence, KV head): its n_q * G (token, head) rows
int32_t priv_tiles(int32_t n_q, int32_t H_q, int32_t H_kv) {
    return ceil_div(static_cast<int64_t>(n_q) * (H_q / std::max(1, H_kv)), 16);
}

// n groups over `pages` pages: the chunk, and the group count that leaves no
// group empty
void cut(int32_t pages, int32_t n, int32_t& chunk, int32_t& groups) {
    n = std::max(1, std::min(n, pages));
    chunk = ceil_div(pages, n);
    groups = ceil_div(pages, chunk);
}

DecodePlan plan_decode(int32_t B, int32_t H_q, int32_t H_kv, int32_t max_pages, int32_t P, int32_t num_splits,
                       int32_t n_q, bool bf16) {
    DecodePlan p;
    if (!bf16) {                                  // the fp32 kernel reads every page per sequence
        const int32_t n = num_splits > 0 ? std::min(num_splits, kMaxSplits) : ceil_div(max_pages, kF32Chunk);
        cut(max_pages, n, p.priv_chunk, p.priv_groups);
        return p;
    }
    const int32_t priv = max_pages - P;
    const int64_t rows = static_cast<int64_t>(B) * n_q * (H_q / std::max(1, H_kv));
    const int64_t tiles = (rows + 15) / 16;
    const int32_t tpw = priv_tiles(n_q, H_q, H_kv) >= 2 ? 2 : 1;       // tiles per wavefront (launcher's rule)
    const int64_t units_v = static_cast<int64_t>(B) * H_kv * ceil_div(priv_tiles(n_q, H_q, H_kv), tpw);
    const int64_t units_p = static_cast<int64_t>(H_kv) * ceil_div(tiles, tpw);
    auto groups_for = [](int64_t units, int32_t pages) {
        const int64_t want = std::max<int64_t>(1, (kTarget + units - 1) / std::max<int64_t>(units, 1));
        return static_cast<int32_t>(std::min<int64_t>(want, std::max(1, pages / kWpg)));
    };
    int32_t gv = 0;
    if (priv > 0) {
        gv = num_splits > 0 ? std::min(num_splits, kMaxSplits) : groups_for(units_v, priv);
        cut(priv, gv, p.priv_chunk, p.priv_groups);
    }
    if (P > 0) {
        int32_t gp = groups_for(units_p, P);
        const int64_t left = kRound - units_v * p.priv_groups;
        gp = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(gp, left / std::max<int64_t>(units_p, 1))));
        cut(P, gp, p.prefix_chunk, p.prefix_groups);
    }
    (void)gv;
    return p;
}

size_t decode_workspace(int64_t rows, int32_t d, int32_t slots) {
    const size_t r = static_cast<size_t>(rows);
    const size_t rs = r * static_cast<size_t>(slots);
    return SPICY_WORKSPACE_HEADER + align_up(4 * r) + align_up(rs * 2 * sizeof(float)) +
           align_up(rs * static_cast<size_t>(d) * sizeof(float));
}

}  // namespace

extern "C" {

const char* spicy_status_string(spicy_status s) {
    switch (s) {
    case SPICY_OK: return "SPICY_OK";
    case SPICY_ERR_ARG: return "SPICY_ERR_ARG: invalid argument";
    case SPICY_ERR_RANGE: return "SPICY_ERR_RANGE: size out of range";
    case SPICY_ERR_CAPACITY: return "SPICY_ERR_CAPACITY: workspace too small";
    case SPICY_ERR_UNSUPPORTED: return "SPICY_ERR_UNSUPPORTED: unsupported shape";
    case SPICY_ERR_HIP: return "SPICY_ERR_HIP: kernel launch failed";
    }
    return "unknown spicy_status";
}

size_t spicy_coarsen_workspace_bytes(int32_t B, int32_t n_seg, int32_t total_tokens, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t dtype) {
    if (B < 0 || n_seg < 0 || total_tokens < 0 || num_kv_heads < 1 || head_dim < 1) return 0;
    if (dtype != SPICY_F32 && dtype != SPICY_BF16) return 0;
    const size_t elem = dtype == SPICY_BF16 ? 2 : 4;
    const size_t ns = static_cast<size_t>(n_seg);
    const size_t nh = ns * static_cast<size_t>(num_kv_heads);
    const size_t items = static_cast<size_t>(total_tokens) * static_cast<size_t>(num_kv_heads);
    const size_t nb = static_cast<size_t>(B);
    const size_t d = static_cast<size_t>(head_dim);
    return SPICY_WORKSPACE_HEADER + align_up(16 * ns) + align_up(8 * nh) + align_up(8 * items) + align_up(4 * nb) +
           align_up(4 * nb * static_cast<size_t>(num_kv_heads)) + 3 * align_up(nh * d * elem) +
           align_up(nh * 2 * elem) + align_up(16 * nh);
}

static spicy_status coarsen_call(const spicy_cache* cache, const void* k_pre, const void* v,
                                 int32_t total_tokens, const int32_t* seq_offsets, const int32_t* pos_base,
                                 const int32_t* seg_offsets, const int32_t* seq_seg_ptr, int32_t n_seg,
                                 const uint8_t* protected_mask, const int64_t* token_weight, int32_t B,
                                 double rope_base, const int32_t* page_table, int32_t max_pages_per_seq,
                                 const int32_t* entry_start, int32_t* lengths_out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    spicy_status st = check_cache(cache);
    if (st != SPICY_OK) return st;
    if (B < 0 || n_seg < 0 || total_tokens < 0) return SPICY_ERR_ARG;
    if (B > kMaxGridY) return SPICY_ERR_UNSUPPORTED;
    if (B == 0) return SPICY_OK;
    if (!seq_offsets || !seg_offsets || !seq_seg_ptr || !page_table || !lengths_out || !workspace)
        return SPICY_ERR_ARG;
    if (total_tokens > 0 && (!k_pre || !v || !protected_mask)) return SPICY_ERR_ARG;
    if (max_pages_per_seq < 1) return SPICY_ERR_ARG;
    if (cache->num_pages < 1) return SPICY_ERR_RANGE;
    if (max_pages_per_seq > kMaxPagesPerSeq) return SPICY_ERR_UNSUPPORTED;
    if (workspace_bytes < spicy_coarsen_workspace_bytes(B, n_seg, total_tokens, cache->num_kv_heads,
                                                        cache->head_dim, cache->dtype))
        return SPICY_ERR_CAPACITY;

    spicy::CoarsenArgs a{};
    a.cache = spicy::CacheArgs{cache->k, cache->v, cache->ab, cache->meta, cache->num_pages, cache->num_kv_heads,
                               cache->s2};
    a.k_pre = k_pre;
    a.v = v;
    a.seq_offsets = seq_offsets;
    a.pos_base = pos_base;
    a.seg_offsets = seg_offsets;
    a.seq_seg_ptr = seq_seg_ptr;
    a.mask = protected_mask;
    a.page_table = page_table;
    a.entry_start = entry_start;
    a.token_weight = total_tokens > 0 ? token_weight : nullptr;
    a.lengths_out = lengths_out;
    char* ws = static_cast<char*>(workspace);
    a.err = reinterpret_cast<int32_t*>(ws);
    const size_t ns = static_cast<size_t>(n_seg);
    a.seg_desc = reinterpret_cast<int4*>(ws + SPICY_WORKSPACE_HEADER);
    size_t off = SPICY_WORKSPACE_HEADER + align_up(16 * ns);
    a.seg_head = reinterpret_cast<int2*>(ws + off);
    // a tag per call for its destination hints (1 .. 2^32 - 1), so that a
    // hint another call published is never taken for this call's
    static std::atomic<uint32_t> calls{0};
    const bool hints = static_cast<int64_t>(n_seg) * cache->num_kv_heads <= spicy::kDestHintWords &&
                       cache->num_pages < (int32_t{1} << 28);
    a.gen = hints ? calls.fetch_add(1, std::memory_order_relaxed) % 0xFFFFFFFFu + 1 : 0u;
    off += align_up(8 * ns * static_cast<size_t>(cache->num_kv_heads));
    a.cp_items = reinterpret_cast<int2*>(ws + off);
    off += align_up(8 * static_cast<size_t>(total_tokens) * static_cast<size_t>(cache->num_kv_heads));
    a.cp_count = reinterpret_cast<int32_t*>(ws + off);
    off += align_up(4 * static_cast<size_t>(B));
    a.null_from = reinterpret_cast<int32_t*>(ws + off);
    off += align_up(4 * static_cast<size_t>(B) * static_cast<size_t>(cache->num_kv_heads));
    const size_t nh = ns * static_cast<size_t>(cache->num_kv_heads);
    const size_t elem = cache->dtype == SPICY_BF16 ? 2 : 4;
    a.stage_k = ws + off;
    off += align_up(nh * static_cast<size_t>(cache->head_dim) * elem);
    a.stage_v = ws + off;
    off += align_up(nh * static_cast<size_t>(cache->head_dim) * elem);
    a.stage_ab = ws + off;
    off += align_up(nh * 2 * elem);
    a.stage_meta = reinterpret_cast<int4*>(ws + off);
    off += align_up(16 * nh);
    a.stage_s2 = ws + off;
    a.total_tokens = total_tokens;
    a.n_seg = n_seg;
    a.B = B;
    a.max_pages = max_pages_per_seq;
    a.rope_base = rope_base;
    for (int i = 0; i < cache->head_dim / 2; ++i)
        a.theta[i] = rope_base > 0.0 ? std::pow(rope_base, -2.0 * static_cast<double>(i) / cache->head_dim) : 0.0;
    return spicy::launch_coarsen(a, cache->dtype, cache->head_dim, static_cast<hipStream_t>(stream));
}

spicy_status spicy_coarsen(const spicy_cache* cache, const void* k_pre, const void* v,
                           int32_t total_tokens, const int32_t* seq_offsets, const int32_t* pos_base,
                           const int32_t* seg_offsets, const int32_t* seq_seg_ptr, int32_t n_seg,
                           const uint8_t* protected_mask, int32_t B, double rope_base,
                           const int32_t* page_table, int32_t max_pages_per_seq,
                           const int32_t* entry_start, int32_t* lengths_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return coarsen_call(cache, k_pre, v, total_tokens, seq_offsets, pos_base, seg_offsets, seq_seg_ptr, n_seg,
                        protected_mask, nullptr, B, rope_base, page_table, max_pages_per_seq, entry_start,
                        lengths_out, workspace, workspace_bytes, stream);
}

spicy_status spicy_coarsen_weighted(const spicy_cache* cache, const void* k_pre, const void* v,
                                    int32_t total_tokens, const int32_t* seq_offsets, const int32_t* pos_base,
                                    const int32_t* seg_offsets, const int32_t* seq_seg_ptr, int32_t n_seg,
                                    const uint8_t* protected_mask, const int64_t* token_weight, int32_t B,
                                    double rope_base, const int32_t* page_table, int32_t max_pages_per_seq,
                                    const int32_t* entry_start, int32_t* lengths_out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (total_tokens > 0 && B > 0 && !token_weight) return SPICY_ERR_ARG;
    return coarsen_call(cache, k_pre, v, total_tokens, seq_offsets, pos_base, seg_offsets, seq_seg_ptr, n_seg,
                        protected_mask, token_weight, B, rope_base, page_table, max_pages_per_seq, entry_start,
                        lengths_out, workspace, workspace_bytes, stream);
}

int32_t spicy_decode_num_splits(int32_t B, int32_t num_kv_heads, int32_t max_pages_per_seq,
                                int32_t num_splits) {
    if (max_pages_per_seq < 1) return 1;
    const int32_t H = std::max(1, num_kv_heads);
    return plan_decode(std::max(B, 0), H, H, max_pages_per_seq, 0, std::max(num_splits, 0), 1, true).priv_groups;
}

spicy_status spicy_decode_plan(int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_pages_per_seq,
                               int32_t shared_prefix_pages, int32_t num_splits, int32_t num_q_tokens,
                               int32_t* plan) {
    if (!plan || B < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_pages_per_seq < 1 || num_q_tokens < 1 ||
        shared_prefix_pages < 0 || num_splits < 0)
        return SPICY_ERR_ARG;
    if (shared_prefix_pages > max_pages_per_seq) return SPICY_ERR_RANGE;
    const DecodePlan p = plan_decode(B, num_q_heads, num_kv_heads, max_pages_per_seq, shared_prefix_pages,
                                     num_splits, num_q_tokens, true);
    plan[0] = p.prefix_groups;
    plan[1] = p.prefix_chunk;
    plan[2] = p.priv_groups;
    plan[3] = p.priv_chunk;
    return SPICY_OK;
}

size_t spicy_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_pages_per_seq, int32_t num_splits) {
    return spicy_decode_shared_workspace_bytes(B, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq, 0,
                                               num_splits);
}

size_t spicy_decode_shared_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_pages_per_seq,
                                           int32_t shared_prefix_pages, int32_t num_splits) {
    return spicy_decode_multi_workspace_bytes(B, 1, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq,
                                              shared_prefix_pages, num_splits);
}

size_t spicy_decode_multi_workspace_bytes(int32_t B, int32_t num_q_tokens, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t max_pages_per_seq,
                                          int32_t shared_prefix_pages, int32_t num_splits) {
    if (B < 0 || num_q_tokens < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
        shared_prefix_pages < 0 || num_splits < 0)
        return 0;
    if (max_pages_per_seq < 1) max_pages_per_seq = 1;
    shared_prefix_pages = std::min(shared_prefix_pages, max_pages_per_seq);
    // reserve for the larger of the bf16 and fp32 plans (the fp32 kernel has
    // no prefix role)
    const DecodePlan p0 = plan_decode(B, num_q_heads, num_kv_heads, max_pages_per_seq, 0, num_splits,
                                      num_q_tokens, false);
    const DecodePlan p1 = plan_decode(B, num_q_heads, num_kv_heads, max_pages_per_seq, shared_prefix_pages,
                                      num_splits, num_q_tokens, true);
    return decode_workspace(static_cast<int64_t>(B) * num_q_tokens * num_q_heads, head_dim,
                            std::max(p0.slots(), p1.slots()));
}

spicy_status spicy_decode_attn(const spicy_cache* cache, const void* q, int32_t num_q_heads,
                               const int32_t* page_table, int32_t max_pages_per_seq,
                               const int32_t* lengths, int32_t B, float* o, float* lse,
                               void* workspace, size_t workspace_bytes, int32_t num_splits,
                               void* stream) {
    return spicy_decode_attn_multi(cache, q, 1, num_q_heads, page_table, max_pages_per_seq, lengths, B, 0, o, lse,
                                   workspace, workspace_bytes, num_splits, stream);
}

spicy_status spicy_decode_attn_shared(const spicy_cache* cache, const void* q, int32_t num_q_heads,
                                      const int32_t* page_table, int32_t max_pages_per_seq,
                                      const int32_t* lengths, int32_t B, int32_t shared_prefix_pages,
                                      float* o, float* lse, void* workspace, size_t workspace_bytes,
                                      int32_t num_splits, void* stream) {
    return spicy_decode_attn_multi(cache, q, 1, num_q_heads, page_table, max_pages_per_seq, lengths, B,
                                   shared_prefix_pages, o, lse, workspace, workspace_bytes, num_splits, stream);
}

}  // extern "C"

namespace {

// Where a decode call keeps its per-row state: the sticky error word (may be
// null), the per-row tickets, and the partial (max, sum) pairs and outputs.
struct DecodeScratch {
    int32_t* err;
    int32_t* ticket;
    float* part_ml;
    float* part_o;
};

// Host checks shared by the decode entry points (nothing launched on error).
spicy_status check_decode(const spicy_cache* cache, const void* q, int32_t num_q_tokens, int32_t num_q_heads,
                          const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* lengths, int32_t B,
                          int32_t shared_prefix_pages, const float* o, const float* lse, int32_t num_splits) {
    spicy_status st = check_cache(cache);
    if (st != SPICY_OK) return st;
    if (B < 0 || num_q_heads < 1 || num_q_tokens < 1 || num_splits < 0 || shared_prefix_pages < 0)
        return SPICY_ERR_ARG;
    if (static_cast<int64_t>(B) * num_q_tokens > kMaxGridY || num_q_heads > kMaxGridY) return SPICY_ERR_UNSUPPORTED;
    if (num_q_heads % cache->num_kv_heads != 0) return SPICY_ERR_UNSUPPORTED;
    if (num_q_heads / cache->num_kv_heads > kMaxGroup) return SPICY_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(B) * num_q_tokens * num_q_heads >= (int64_t(1) << 31) / kMaxGroup)
        return SPICY_ERR_UNSUPPORTED;
    if (B == 0) return SPICY_OK;
    if (!q || !page_table || !lengths || !o || !lse) return SPICY_ERR_ARG;
    if (max_pages_per_seq < 1) return SPICY_ERR_ARG;
    if (shared_prefix_pages > max_pages_per_seq) return SPICY_ERR_RANGE;
    return SPICY_OK;
}

spicy_status decode_launch(const spicy_cache* cache, const void* q, int32_t num_q_tokens, int32_t num_q_heads,
                           const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* lengths, int32_t B,
                           int32_t shared_prefix_pages, float* o, float* lse, const DecodeScratch& sc,
                           const DecodePlan& plan, int32_t P, void* stream) {
    spicy::DecodeArgs a{};
    a.cache = spicy::CacheArgs{cache->k, cache->v, cache->ab, cache->meta, cache->num_pages, cache->num_kv_heads,
                               cache->s2};
    a.q = q;
    a.page_table = page_table;
    a.lengths = lengths;
    a.o = o;
    a.lse = lse;
    a.err = sc.err;
    a.ticket = sc.ticket;
    a.part_ml = sc.part_ml;
    a.part_o = sc.part_o;
    a.B = B;
    a.H_q = num_q_heads;
    a.max_pages = max_pages_per_seq;
    a.n_q = num_q_tokens;
    a.slots = plan.slots();
    a.prefix_pages = P;
    a.prefix_groups = plan.prefix_groups;
    a.prefix_chunk = plan.prefix_chunk;
    a.priv_groups = plan.priv_groups;
    a.priv_chunk = plan.priv_chunk;
    a.priv_tiles = priv_tiles(num_q_tokens, num_q_heads, cache->num_kv_heads);
    a.wpg = plan.wpg;
    return spicy::launch_decode(a, cache->dtype, cache->head_dim, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------ the no-allocation decode

// The decode scratch of spicy_decode_attn_multi_noalloc: one array per GPU,
// in the library's code object (zero when the library loads; every call
// leaves its tickets at zero).  Layout: [0, 256) unused header; the tickets
// of up to kNoAllocMaxRows query rows at a fixed place, so that calls of any
// shape find theirs at zero; then the partials of the call.
constexpr size_t kNoAllocBytes = size_t(32) << 20;
constexpr int64_t kNoAllocMaxRows = 65536;
constexpr size_t kNoAllocTickets = SPICY_WORKSPACE_HEADER;
constexpr size_t kNoAllocPartials = SPICY_WORKSPACE_HEADER + 4 * kNoAllocMaxRows;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];        // per device: scratch's device address (from hipGetSymbolAddress)

// The scratch address on the current device, looked up once per device with
// that device current; nullptr if the lookup fails.
void* scratch_on_current_device(int* dev_out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    *dev_out = dev;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

spicy_status spicy_decode_attn_multi(const spicy_cache* cache, const void* q, int32_t num_q_tokens,
                                     int32_t num_q_heads, const int32_t* page_table, int32_t max_pages_per_seq,
                                     const int32_t* lengths, int32_t B, int32_t shared_prefix_pages, float* o,
                                     float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits,
                                     void* stream) {
    spicy_status st = check_decode(cache, q, num_q_tokens, num_q_heads, page_table, max_pages_per_seq, lengths, B,
                                   shared_prefix_pages, o, lse, num_splits);
    if (st != SPICY_OK || B == 0) return st;
    if (!workspace) return SPICY_ERR_ARG;
    if (workspace_bytes < spicy_decode_multi_workspace_bytes(B, num_q_tokens, num_q_heads, cache->num_kv_heads,
                                                             cache->head_dim, max_pages_per_seq,
                                                             shared_prefix_pages, num_splits))
        return SPICY_ERR_CAPACITY;
    // the fp32 kernel has no shared-prefix role: every page is private there
    const bool bf16 = cache->dtype == SPICY_BF16;
    const int32_t P = bf16 ? shared_prefix_pages : 0;
    const DecodePlan plan = plan_decode(B, num_q_heads, cache->num_kv_heads, max_pages_per_seq, P, num_splits,
                                        num_q_tokens, bf16);
    char* ws = static_cast<char*>(workspace);
    const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(num_q_tokens) *
                        static_cast<size_t>(num_q_heads);
    DecodeScratch sc;
    sc.err = reinterpret_cast<int32_t*>(ws);
    size_t off = SPICY_WORKSPACE_HEADER;
    sc.ticket = reinterpret_cast<int32_t*>(ws + off);
    off += align_up(4 * rows);
    sc.part_ml = reinterpret_cast<float*>(ws + off);
    off += align_up(rows * static_cast<size_t>(plan.slots()) * 2 * sizeof(float));
    sc.part_o = reinterpret_cast<float*>(ws + off);
    return decode_launch(cache, q, num_q_tokens, num_q_heads, page_table, max_pages_per_seq, lengths, B,
                         shared_prefix_pages, o, lse, sc, plan, P, stream);
}

size_t spicy_decode_noalloc_max_bytes(void) { return kNoAllocBytes; }

spicy_status spicy_decode_attn_multi_noalloc(const spicy_cache* cache, const void* q, int32_t num_q_tokens,
                                             int32_t num_q_heads, const int32_t* page_table,
                                             int32_t max_pages_per_seq, const int32_t* lengths, int32_t B,
                                             int32_t shared_prefix_pages, float* o, float* lse,
                                             int32_t* device_error, int32_t num_splits, void* stream) {
    spicy_status st = check_decode(cache, q, num_q_tokens, num_q_heads, page_table, max_pages_per_seq, lengths, B,
                                   shared_prefix_pages, o, lse, num_splits);
    if (st != SPICY_OK || B == 0) return st;
    const bool bf16 = cache->dtype == SPICY_BF16;
    const int32_t P = bf16 ? shared_prefix_pages : 0;
    const DecodePlan plan = plan_decode(B, num_q_heads, cache->num_kv_heads, max_pages_per_seq, P, num_splits,
                                        num_q_tokens, bf16);
    const int64_t rows = static_cast<int64_t>(B) * num_q_tokens * num_q_heads;
    const size_t rs = static_cast<size_t>(rows) * static_cast<size_t>(plan.slots());
    const size_t ml_bytes = align_up(rs * 2 * sizeof(float));
    if (rows > kNoAllocMaxRows ||
        kNoAllocPartials + ml_bytes + rs * static_cast<size_t>(cache->head_dim) * sizeof(float) > kNoAllocBytes)
        return SPICY_ERR_CAPACITY;
    // the stream must run on the current device, whose scratch the call uses
    int dev = -1;
    char* base = static_cast<char*>(scratch_on_current_device(&dev));
    if (!base) return SPICY_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return SPICY_ERR_HIP;
        if (sdev != dev) return SPICY_ERR_ARG;
    }
    DecodeScratch sc;
    sc.err = device_error;
    sc.ticket = reinterpret_cast<int32_t*>(base + kNoAllocTickets);
    sc.part_ml = reinterpret_cast<float*>(base + kNoAllocPartials);
    sc.part_o = reinterpret_cast<float*>(base + kNoAllocPartials + ml_bytes);
    return decode_launch(cache, q, num_q_tokens, num_q_heads, page_table, max_pages_per_seq, lengths, B,
                         shared_prefix_pages, o, lse, sc, plan, P, stream);
}

size_t spicy_policy_workspace_bytes(int32_t total_tokens, int32_t num_kv_heads) {
    if (total_tokens < 0 || num_kv_heads < 1) return 0;
    const size_t T = static_cast<size_t>(total_tokens);
    return SPICY_WORKSPACE_HEADER + align_up(8 * T) + align_up(8 * T * static_cast<size_t>(num_kv_heads));
}

spicy_status spicy_policy(const void* k_pre, const void* v, int32_t total_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t dtype, const int32_t* seq_offsets, int32_t B,
                          const int32_t* proj_ptr, const int32_t* proj_idx, int32_t proj_rows, int32_t proj_nnz,
                          int32_t n_segments, int32_t n_landmarks, int32_t sink, int32_t recent,
                          int32_t* seg_offsets, int32_t* seq_seg_ptr, uint8_t* protected_mask, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (dtype != SPICY_BF16 && dtype != SPICY_F32) return SPICY_ERR_ARG;
    if (dtype != SPICY_BF16) return SPICY_ERR_UNSUPPORTED;
    if (!head_dim_ok(head_dim)) return SPICY_ERR_UNSUPPORTED;
    if (num_kv_heads < 1 || num_kv_heads > kMaxKvHeads) return SPICY_ERR_UNSUPPORTED;
    if (total_tokens < 0 || B < 0 || proj_nnz < 0 || n_segments < 1 || n_landmarks < 0 || sink < 0 ||
        recent < 0 || proj_rows < 1 || proj_rows > 16)
        return SPICY_ERR_ARG;
    if (static_cast<int64_t>(B) * n_segments + 1 > INT32_MAX) return SPICY_ERR_ARG;
    if (B > kMaxGridY) return SPICY_ERR_UNSUPPORTED;
    if (B == 0) return SPICY_OK;
    if (!k_pre || !v || !seq_offsets || !proj_ptr || (proj_nnz > 0 && !proj_idx) || !seg_offsets ||
        !seq_seg_ptr || !protected_mask || !workspace)
        return SPICY_ERR_ARG;
    if (workspace_bytes < spicy_policy_workspace_bytes(total_tokens, num_kv_heads)) return SPICY_ERR_CAPACITY;

    spicy::PolicyArgs a{};
    a.k = static_cast<const uint16_t*>(k_pre);
    a.v = static_cast<const uint16_t*>(v);
    a.seq_offsets = seq_offsets;
    a.proj_ptr = proj_ptr;
    a.proj_idx = proj_idx;
    a.seg_offsets = seg_offsets;
    a.seq_seg_ptr = seq_seg_ptr;
    a.mask = protected_mask;
    char* ws = static_cast<char*>(workspace);
    a.err = reinterpret_cast<int32_t*>(ws);
    size_t off = SPICY_WORKSPACE_HEADER;
    a.var = reinterpret_cast<int64_t*>(ws + off);
    off += align_up(8 * static_cast<size_t>(total_tokens));
    a.norm2 = reinterpret_cast<uint64_t*>(ws + off);
    a.total_tokens = total_tokens;
    a.B = B;
    a.H = num_kv_heads;
    a.d = head_dim;
    a.R = proj_rows;
    a.nnz = proj_nnz;
    a.N = n_segments;
    a.L = n_landmarks;
    a.sink = sink;
    a.recent = recent;
    return spicy::launch_policy(a, static_cast<hipStream_t>(stream));
}

size_t spicy_merge_workspace_bytes(int32_t B, int32_t num_kv_heads, int32_t max_range) {
    if (B < 0 || num_kv_heads < 1 || max_range < 0) return 0;
    const size_t units = static_cast<size_t>(B) * static_cast<size_t>(num_kv_heads);
    return SPICY_WORKSPACE_HEADER + align_up(4 * units);
}

spicy_status spicy_merge_level(const spicy_cache* cache, int32_t B, double rope_base, const int32_t* page_table,
                               int32_t max_pages_per_seq, const int32_t* entry_begin, const int32_t* entry_end,
                               int32_t max_range, void* workspace, size_t workspace_bytes, void* stream) {
    spicy_status st = check_cache(cache);
    if (st != SPICY_OK) return st;
    if (B < 0 || max_range < 0) return SPICY_ERR_ARG;
    if (!cache->meta) return SPICY_ERR_ARG;              // the exact masses and anchors live there
    if (cache->s2) return SPICY_ERR_UNSUPPORTED;         // per-dimension variances do not merge from the diagonal
    if (B == 0) return SPICY_OK;
    if (!page_table || !entry_begin || !entry_end || !workspace) return SPICY_ERR_ARG;
    if (max_pages_per_seq < 1) return SPICY_ERR_ARG;
    if (static_cast<int64_t>(B) * cache->num_kv_heads > kMaxGridY) return SPICY_ERR_UNSUPPORTED;
    if (workspace_bytes < spicy_merge_workspace_bytes(B, cache->num_kv_heads, max_range)) return SPICY_ERR_CAPACITY;
    spicy::MergeArgs a{};
    a.cache = spicy::CacheArgs{cache->k, cache->v, cache->ab, cache->meta, cache->num_pages, cache->num_kv_heads,
                               cache->s2};
    a.page_table = page_table;
    a.entry_begin = entry_begin;
    a.entry_end = entry_end;
    char* ws = static_cast<char*>(workspace);
    a.err = reinterpret_cast<int32_t*>(ws);
    a.ticket = reinterpret_cast<int32_t*>(ws + SPICY_WORKSPACE_HEADER);
    a.cap = static_cast<int32_t>((static_cast<int64_t>(max_range) + 1) / 2);
    a.B = B;
    a.max_pages = max_pages_per_seq;
    a.max_range = max_range;
    a.rope_base = rope_base;
    for (int i = 0; i < cache->head_dim / 2; ++i)
        a.theta[i] = rope_base > 0.0 ? std::pow(rope_base, -2.0 * static_cast<double>(i) / cache->head_dim) : 0.0;
    return spicy::launch_merge(a, cache->dtype, cache->head_dim, static_cast<hipStream_t>(stream));
}

spicy_status spicy_compact_range(const spicy_cache* cache, int32_t B, const int32_t* page_table,
                                 int32_t max_pages_per_seq, const int32_t* entry_begin, const int32_t* lengths,
                                 int32_t* lengths_out, int32_t* device_error, void* stream) {
    spicy_status st = check_cache(cache);
    if (st != SPICY_OK) return st;
    if (B < 0) return SPICY_ERR_ARG;
    if (B == 0) return SPICY_OK;
    if (!page_table || !entry_begin || !lengths || !lengths_out || !device_error) return SPICY_ERR_ARG;
    if (max_pages_per_seq < 1) return SPICY_ERR_ARG;
    // the move launch reads entry_begin and lengths after the count launch
    // has written lengths_out
    if (lengths_out == lengths || lengths_out == entry_begin) return SPICY_ERR_ARG;
    if (B > kMaxGridY) return SPICY_ERR_UNSUPPORTED;
    spicy::CompactArgs a{};
    a.cache = spicy::CacheArgs{cache->k, cache->v, cache->ab, cache->meta, cache->num_pages, cache->num_kv_heads,
                               cache->s2};
    a.page_table = page_table;
    a.entry_begin = entry_begin;
    a.lengths = lengths;
    a.lengths_out = lengths_out;
    a.err = device_error;
    a.B = B;
    a.max_pages = max_pages_per_seq;
    a.D = cache->head_dim;
    return spicy::launch_compact(a, cache->dtype, static_cast<hipStream_t>(stream));
}

}  // extern "C"
