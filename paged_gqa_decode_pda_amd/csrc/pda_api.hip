// Host side of the C ABI declared in include/pda.h: argument validation, split
// planning and kernel launches.  Nothing here allocates device memory or
// synchronises (the one device array, pda_decode_noalloc's scratch, has
// static storage); every check runs before the first enqueue.
#include "../../include/pda.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "pda_internal.h"
#include "pda_rope.h"

struct pda_plan {
    pda_dims dims;
    float *m, *l, *o;
    void *workspace;
    size_t workspace_bytes;
    int32_t bps_request;
};

namespace {

thread_local char g_err[512];

pda_status fail(pda_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

void clear_err() { g_err[0] = 0; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Bytes rounded up to a multiple of 16 (the start of every region the
// kernels read or write with 16-byte accesses).
size_t round16(size_t n) { return (n + 15) & ~size_t(15); }

pda_status check_dims(const pda_dims *d) {
    if (!d) return fail(PDA_ERR_NULL, "dims is NULL");
    if (d->max_seqs < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 ||
        d->block_size < 1 || d->tile_capacity < 1)
        return fail(PDA_ERR_DIMS, "every dimension must be >= 1");
    if (d->num_q_heads % d->num_kv_heads != 0)
        return fail(PDA_ERR_GQA, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                    d->num_q_heads, d->num_kv_heads);
    if (d->head_dim > 256) return fail(PDA_ERR_HEAD_DIM, "head_dim %d exceeds 256", d->head_dim);
    if (d->head_dim % 8 != 0)
        return fail(PDA_ERR_HEAD_DIM, "head_dim %d is not a multiple of 8", d->head_dim);
    const int64_t tile_tokens = (int64_t)d->tile_capacity * d->block_size;
    if (tile_tokens > (int64_t(1) << 24) ||
        (uint64_t)tile_tokens * (uint64_t)d->block_size > (uint64_t(1) << 32))
        return fail(PDA_ERR_DIMS, "tile_capacity * block_size too large");
    const int64_t G = d->num_q_heads / d->num_kv_heads;
    const pda::Plan p = pda::choose_plan((int)G, d->head_dim, d->block_size);
    if ((int64_t)d->num_kv_heads * p.nhc > 65535 || d->max_seqs > 65535)
        return fail(PDA_ERR_DIMS, "num_kv_heads * head chunks and max_seqs must be <= 65535");
    return PDA_OK;
}

int32_t min_auto_bps(const pda_dims *d) {
    const int32_t lo = (int32_t)ceil_div(d->tile_capacity, 256);
    return lo < 1 ? 1 : lo;
}

int device_cus() {
    // queried once per device (the count does not change while the process runs)
    static std::atomic<int> known[64];   // 0: not yet queried
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    const bool slot = dev >= 0 && dev < 64;
    if (slot && (cus = known[dev].load(std::memory_order_relaxed)) > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return 256;
    if (slot) known[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Events armed by pda_debug_time_attention for this thread's next launch.
thread_local pda::AttendEvents t_events;

pda::AttendEvents take_events() {
    const pda::AttendEvents ev = t_events;
    t_events = pda::AttendEvents{};
    return ev;
}

// Pages per split.  An explicit request is clamped to [1, tile_capacity].
// Otherwise splits of about 256 tokens (16 groups of 16), 352 at head dims
// above 128, never more than 256 splits per sequence.  (Measured on MI355X:
// at head dim 128, 256 tokens beat 320 and 384 on the ragged and small
// batches; at head dim 256, 352 tokens ran the 8-tile, 4-sequence workload
// 3 % faster than 256, and 320 or 384 in between the two.)
int32_t resolve_bps(const pda_dims *d, int32_t request, int32_t num_seqs) {
    (void)num_seqs;
    const int32_t cap = d->tile_capacity;
    if (request > 0) return request > cap ? cap : request;
    int32_t bps = (d->head_dim > 128 ? 352 : 256) / d->block_size;
    if (bps < 1) bps = 1;
    if (bps < min_auto_bps(d)) bps = min_auto_bps(d);
    if (bps > cap) bps = cap;
    return bps;
}

// Partial slots one (sequence, q head) row can need: one per item.  A
// sequence of n splits has n items when every split is an item, and
// n - (big - 1) * floor(e n / (8 big)) with big items (never more), so n
// bounds both sizings the attention kernel may choose.
int64_t slots_per_seq(const pda_dims *d, int32_t bps) {
    return ceil_div(d->tile_capacity, bps);
}

int64_t units_of(const pda_dims *d) {
    const int G = d->num_q_heads / d->num_kv_heads;
    return (int64_t)d->num_kv_heads * pda::choose_plan(G, d->head_dim, d->block_size).nhc;
}

// The decode workspace: control words, the arrival counters (one 64-bit word
// per (sequence, unit)), then the split partials for max_seqs sequences:
// (m, l) pairs, padded to 16 bytes, then o rows.
size_t arrive_bytes(const pda_dims *d) { return round16((size_t)d->max_seqs * units_of(d) * 8); }

// (m, l) pairs of the partials, in floats, padded to 16 bytes so the o rows
// after them start 16-byte aligned.
size_t partial_ml_floats(const pda_dims *d, int32_t bps) {
    return round16((size_t)d->max_seqs * d->num_q_heads * slots_per_seq(d, bps) * 2 * sizeof(float)) /
           sizeof(float);
}

// A unit's partial o rows (its q heads, every split slot) must span less than
// 2 GiB: the kernel addresses them with 32-bit offsets from the unit's start.
pda_status check_partial_span(const pda_dims *d, int32_t bps) {
    const int G = d->num_q_heads / d->num_kv_heads;
    const int64_t heads = G < pda::kHeadsPerItem ? G : pda::kHeadsPerItem;
    if (heads * slots_per_seq(d, bps) * d->head_dim * 4 >= (int64_t(1) << 31))
        return fail(PDA_ERR_DIMS, "%lld split slots per sequence (tile_capacity / blocks_per_split) are too many",
                    (long long)slots_per_seq(d, bps));
    return PDA_OK;
}

size_t workspace_for(const pda_dims *d, int32_t bps) {
    return (size_t)pda::kCtrlBytes + arrive_bytes(d) + partial_ml_floats(d, bps) * sizeof(float) +
           (size_t)d->max_seqs * d->num_q_heads * slots_per_seq(d, bps) * d->head_dim * sizeof(float);
}

// Launch epochs: each attention launch tags the workspace counters with its
// own 32-bit value.  The sequence starts at a value drawn from the clock when
// the library is loaded, so launches of this process do not meet epochs that a
// previous user of the same memory left behind (other than by a 2^-32 chance).
std::atomic<uint32_t> g_epoch{(uint32_t)(std::chrono::steady_clock::now().time_since_epoch().count() *
                                         0x9E3779B97F4A7C15ull >> 32)};

uint32_t next_epoch() { return g_epoch.fetch_add(1, std::memory_order_relaxed) + 1; }

pda_status check_strides(const pda_dims *d, pda_strides st) {
    if (st.blk < 0 || st.tok < 0 || st.kvh < 0)
        return fail(PDA_ERR_ALIGN, "strides must be non-negative");
    if (st.blk % 8 || st.tok % 8 || st.kvh % 8)
        return fail(PDA_ERR_ALIGN, "strides (%lld, %lld, %lld) must be multiples of 8 elements",
                    (long long)st.blk, (long long)st.tok, (long long)st.kvh);
    // below 2^32 each, a 32-bit page id times the page stride fits 64 bits
    if (st.blk >= (int64_t(1) << 32) || st.tok >= (int64_t(1) << 32) || st.kvh >= (int64_t(1) << 32))
        return fail(PDA_ERR_DIMS, "strides (%lld, %lld, %lld) must be below 2^32 elements",
                    (long long)st.blk, (long long)st.tok, (long long)st.kvh);
    const __int128 in_page = (__int128)(d->block_size - 1) * st.tok +
                             (__int128)(d->num_kv_heads - 1) * st.kvh + d->head_dim;
    if (in_page >= (__int128(1) << 31))
        return fail(PDA_ERR_DIMS, "a token row offset inside a page exceeds 2^31 elements");
    return PDA_OK;
}

pda_status check_tile_ptrs(const void *q, const void *k, const void *v, const int32_t *blocks,
                           const int32_t *counts, const int32_t *lastv) {
    if (!q || !k || !v || !blocks || !counts) return fail(PDA_ERR_NULL, "a required pointer is NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(PDA_ERR_ALIGN, "q, k_pool and v_pool must be 16-byte aligned");
    if (!aligned(blocks, 4) || !aligned(counts, 4) || (lastv && !aligned(lastv, 4)))
        return fail(PDA_ERR_ALIGN, "page-id, count and last-valid arrays must be 4-byte aligned");
    return PDA_OK;
}

pda::AttendArgs attend_args(const pda_dims *d, const void *q, const void *k, const void *v,
                            const int32_t *blocks, const int32_t *counts, const int32_t *lastv,
                            int32_t lv_default, pda_strides st, int32_t bps, void *ws, int S,
                            const pda::Plan &p) {
    pda::AttendArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.blocks = blocks;
    a.counts = counts;
    a.lastv = lastv;
    a.blk = st.blk;
    a.tok = st.tok;
    a.kvh = st.kvh;
    a.bs_magic = ((uint64_t(1) << 32) + (uint64_t)d->block_size - 1) / (uint64_t)d->block_size;
    a.S = S;
    a.Hq = d->num_q_heads;
    a.Hkv = d->num_kv_heads;
    a.G = d->num_q_heads / d->num_kv_heads;
    a.D = d->head_dim;
    a.bs = d->block_size;
    a.cap = d->tile_capacity;
    a.bps = bps;
    a.nhc = p.nhc;
    a.nsplit = (int32_t)slots_per_seq(d, bps);   // partial slots per (sequence, q head)
    a.lv_default = lv_default;
    a.prefix_mode = S <= pda::kPrefixMaxSeqs ? 1 : 0;
    a.epoch = next_epoch();
    // Test knob: without the restart pass of a launch that makes claims,
    // every counter the launch finds with another epoch is restarted by its
    // first claim or arrival (the path that launches without claims always
    // take for arrivals, and claims only in a race with the pass).
    a.restart = std::getenv("PDA_DEBUG_NO_COUNTER_RESTART") ? 0 : 1;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
    char *wsb = static_cast<char *>(ws);
    a.work = reinterpret_cast<unsigned long long *>(wsb);
    a.arrive = reinterpret_cast<unsigned long long *>(wsb + pda::kCtrlBytes);
    float *wsf = reinterpret_cast<float *>(wsb + pda::kCtrlBytes + arrive_bytes(d));
    a.part_ml = wsf;
    a.part_o = wsf + partial_ml_floats(d, bps);
    a.out = nullptr;
    a.m = a.l = a.o = nullptr;
    a.mask = nullptr;
    a.mask_stride = 0;
    return a;
}

pda_status hip_fail(hipError_t e, const char *what) {
    return fail(PDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The workspace of pda_decode_noalloc: a device array with static storage,
// one copy per GPU the library runs on (created with the code object on that
// device, zero at load, held until the process ends).  Host code never uses
// the array's name as an address (on the host it is only a stand-in for the
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[PDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device).
pda_status noalloc_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PDA_ERR_DIMS, "device %d is beyond the %d devices the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(PDA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return PDA_OK;
}

}  // namespace

extern "C" {

pda_status pda_dims_validate(const pda_dims *dims) {
    clear_err();
    return check_dims(dims);
}

size_t pda_state_bytes(const pda_dims *d) {
    if (check_dims(d) != PDA_OK) return 0;
    const size_t rows = (size_t)d->max_seqs * d->num_q_heads;
    return 2 * round16(rows * sizeof(float)) + rows * sizeof(float) * (size_t)d->head_dim;
}

pda_status pda_state_offsets(const pda_dims *d, size_t offsets[3]) {
    clear_err();
    pda_status st = check_dims(d);
    if (st != PDA_OK) return st;
    if (!offsets) return fail(PDA_ERR_NULL, "offsets is NULL");
    const size_t rows = (size_t)d->max_seqs * d->num_q_heads;
    offsets[0] = 0;
    offsets[1] = round16(rows * sizeof(float));
    offsets[2] = 2 * round16(rows * sizeof(float));
    return PDA_OK;
}

int32_t pda_blocks_per_split(const pda_dims *d, int32_t request) {
    if (check_dims(d) != PDA_OK) return 0;
    return resolve_bps(d, request, d->max_seqs);
}

size_t pda_workspace_bytes(const pda_dims *d, int32_t request) {
    if (check_dims(d) != PDA_OK) return 0;
    const int32_t bps = request > 0 ? (request > d->tile_capacity ? d->tile_capacity : request)
                                    : min_auto_bps(d);
    return workspace_for(d, bps);
}

pda_strides pda_paged_strides(const pda_dims *d) {
    pda_strides s{0, 0, 0};
    if (!d) return s;
    s.blk = (int64_t)d->block_size * d->num_kv_heads * d->head_dim;
    s.tok = (int64_t)d->num_kv_heads * d->head_dim;
    s.kvh = d->head_dim;
    return s;
}

pda_strides pda_scratch_pool_strides(const pda_dims *d) {
    pda_strides s{0, 0, 0};
    if (!d) return s;
    const int64_t stripe = (int64_t)d->num_kv_heads * d->block_size * d->head_dim;
    s.blk = 2 * stripe;
    s.tok = d->head_dim;
    s.kvh = (int64_t)d->block_size * d->head_dim;
    return s;
}

int64_t pda_scratch_pool_v_offset(const pda_dims *d) {
    if (!d) return 0;
    return (int64_t)d->num_kv_heads * d->block_size * d->head_dim;
}

pda_status pda_create(const pda_dims *dims, void *state, void *workspace, size_t workspace_bytes,
                      int32_t blocks_per_split, pda_plan **out) {
    clear_err();
    pda_status st = check_dims(dims);
    if (st != PDA_OK) return st;
    if (!state || !out) return fail(PDA_ERR_NULL, "state and out must be non-NULL");
    if (!aligned(state, 16)) return fail(PDA_ERR_ALIGN, "state must be 16-byte aligned");
    if (blocks_per_split < 0) return fail(PDA_ERR_DIMS, "blocks_per_split must be >= 0");
    if (workspace && !aligned(workspace, 16))
        return fail(PDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t need = pda_workspace_bytes(dims, blocks_per_split);
    if (!workspace || workspace_bytes < need)
        return fail(PDA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
    pda_plan *p = new (std::nothrow) pda_plan;
    if (!p) return fail(PDA_ERR_DIMS, "out of host memory");
    p->dims = *dims;
    const size_t rows = (size_t)dims->max_seqs * dims->num_q_heads;
    const size_t mlen = round16(rows * sizeof(float)) / sizeof(float);   // m and l, each padded to 16 bytes
    p->m = static_cast<float *>(state);
    p->l = p->m + mlen;
    p->o = p->l + mlen;
    p->workspace = workspace;
    p->workspace_bytes = workspace_bytes;
    p->bps_request = blocks_per_split;
    *out = p;
    return PDA_OK;
}

void pda_destroy(pda_plan *plan) { delete plan; }

pda_status pda_begin_step(pda_plan *plan, int32_t num_seqs, void *stream) {
    clear_err();
    if (!plan) return fail(PDA_ERR_NULL, "plan is NULL");
    if (num_seqs < 0 || num_seqs > plan->dims.max_seqs)
        return fail(PDA_ERR_MAX_SEQS, "begin_step num_seqs %d outside [0, max_seqs=%d]", num_seqs,
                    plan->dims.max_seqs);
    if (num_seqs == 0) return PDA_OK;
    hipError_t e = pda::launch_reset(plan->m, plan->l, plan->o,
                                     (int64_t)num_seqs * plan->dims.num_q_heads, plan->dims.head_dim,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PDA_OK : hip_fail(e, "reset launch");
}

pda_status pda_step_tile(pda_plan *plan, const void *q, const void *k_pool, const void *v_pool,
                         const int32_t *tile_blocks, const int32_t *tile_block_counts,
                         const int32_t *last_block_valid, int32_t last_block_valid_default,
                         int32_t num_seqs, pda_strides strides, void *stream) {
    clear_err();
    if (!plan) return fail(PDA_ERR_NULL, "plan is NULL");
    const pda_dims *d = &plan->dims;
    if (num_seqs < 0 || num_seqs > d->max_seqs)
        return fail(PDA_ERR_MAX_SEQS, "num_seqs %d outside [0, max_seqs=%d]", num_seqs, d->max_seqs);
    pda_status st = check_tile_ptrs(q, k_pool, v_pool, tile_blocks, tile_block_counts, last_block_valid);
    if (st != PDA_OK) return st;
    if ((st = check_strides(d, strides)) != PDA_OK) return st;
    if (num_seqs == 0) return PDA_OK;
    const int32_t bps = resolve_bps(d, plan->bps_request, num_seqs);
    if ((st = check_partial_span(d, bps)) != PDA_OK) return st;
    if (workspace_for(d, bps) > plan->workspace_bytes)
        return fail(PDA_ERR_WORKSPACE, "workspace too small");
    const int G = d->num_q_heads / d->num_kv_heads;
    const pda::Plan p = pda::choose_plan(G, d->head_dim, d->block_size);
    pda::AttendArgs a = attend_args(d, q, k_pool, v_pool, tile_blocks, tile_block_counts,
                                    last_block_valid, last_block_valid_default, strides, bps,
                                    plan->workspace, num_seqs, p);
    a.m = plan->m;
    a.l = plan->l;
    a.o = plan->o;
    hipError_t e = pda::launch_attend(p, a, device_cus(), static_cast<hipStream_t>(stream), take_events());
    return e == hipSuccess ? PDA_OK : hip_fail(e, "tile launch");
}

pda_status pda_finalize(pda_plan *plan, void *out, int32_t num_seqs, void *stream) {
    clear_err();
    if (!plan) return fail(PDA_ERR_NULL, "plan is NULL");
    if (num_seqs < 0 || num_seqs > plan->dims.max_seqs)
        return fail(PDA_ERR_MAX_SEQS, "num_seqs %d outside [0, max_seqs=%d]", num_seqs,
                    plan->dims.max_seqs);
    if (!out) return fail(PDA_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(PDA_ERR_ALIGN, "out must be 16-byte aligned");
    if (num_seqs == 0) return PDA_OK;
    hipError_t e = pda::launch_finalize(plan->l, plan->o, static_cast<uint16_t *>(out),
                                        (int64_t)num_seqs * plan->dims.num_q_heads,
                                        plan->dims.head_dim, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PDA_OK : hip_fail(e, "finalize launch");
}

namespace {

pda_status decode_impl(const pda_dims *dims, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *block_tables, const int32_t *block_counts,
                       const int32_t *last_block_valid, int32_t last_block_valid_default,
                       int32_t num_seqs, pda_strides strides, const uint8_t *kv_mask,
                       int64_t mask_stride, void *workspace, size_t workspace_bytes, void *out,
                       int32_t blocks_per_split, void *stream, bool noalloc = false) {
    pda_status st = check_dims(dims);
    if (st != PDA_OK) return st;
    if (num_seqs < 0 || num_seqs > dims->max_seqs)
        return fail(PDA_ERR_MAX_SEQS, "num_seqs %d outside [0, max_seqs=%d]", num_seqs, dims->max_seqs);
    if (blocks_per_split < 0) return fail(PDA_ERR_DIMS, "blocks_per_split must be >= 0");
    if ((st = check_tile_ptrs(q, k_pool, v_pool, block_tables, block_counts, last_block_valid)) != PDA_OK)
        return st;
    if (!out) return fail(PDA_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(PDA_ERR_ALIGN, "out must be 16-byte aligned");
    if ((st = check_strides(dims, strides)) != PDA_OK) return st;
    if (workspace && !aligned(workspace, 16))
        return fail(PDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    const int32_t bps = resolve_bps(dims, blocks_per_split, num_seqs);
    if ((st = check_partial_span(dims, bps)) != PDA_OK) return st;
    const size_t need = workspace_for(dims, bps);
    if (noalloc && need > PDA_NOALLOC_SCRATCH_BYTES)
        return fail(PDA_ERR_WORKSPACE,
                    "pda_decode_noalloc needs %zu bytes of scratch for these dims and %d pages per "
                    "split; its built-in scratch holds %zu (raise blocks_per_split, lower max_seqs "
                    "or tile_capacity, or call pda_decode with a workspace)",
                    need, bps, (size_t)PDA_NOALLOC_SCRATCH_BYTES);
    if (num_seqs == 0) return PDA_OK;
    if (noalloc) {
        if ((st = noalloc_scratch(&workspace)) != PDA_OK) return st;
        workspace_bytes = PDA_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need)
        return fail(PDA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
    const int G = dims->num_q_heads / dims->num_kv_heads;
    const pda::Plan p = pda::choose_plan(G, dims->head_dim, dims->block_size);
    pda::AttendArgs a = attend_args(dims, q, k_pool, v_pool, block_tables, block_counts,
                                    last_block_valid, last_block_valid_default, strides, bps,
                                    workspace, num_seqs, p);
    a.out = static_cast<uint16_t *>(out);
    a.mask = kv_mask;
    a.mask_stride = mask_stride;
    hipError_t e = pda::launch_attend(p, a, device_cus(), static_cast<hipStream_t>(stream), take_events());
    return e == hipSuccess ? PDA_OK : hip_fail(e, "decode launch");
}

}  // namespace

pda_status pda_decode(const pda_dims *dims, const void *q, const void *k_pool, const void *v_pool,
                      const int32_t *block_tables, const int32_t *block_counts,
                      const int32_t *last_block_valid, int32_t last_block_valid_default,
                      int32_t num_seqs, pda_strides strides, void *workspace,
                      size_t workspace_bytes, void *out, int32_t blocks_per_split, void *stream) {
    clear_err();
    return decode_impl(dims, q, k_pool, v_pool, block_tables, block_counts, last_block_valid,
                       last_block_valid_default, num_seqs, strides, nullptr, 0, workspace,
                       workspace_bytes, out, blocks_per_split, stream);
}

pda_status pda_decode_noalloc(const pda_dims *dims, const void *q, const void *k_pool,
                              const void *v_pool, const int32_t *block_tables,
                              const int32_t *block_counts, const int32_t *last_block_valid,
                              int32_t last_block_valid_default, int32_t num_seqs,
                              pda_strides strides, void *out, int32_t blocks_per_split,
                              void *stream) {
    clear_err();
    return decode_impl(dims, q, k_pool, v_pool, block_tables, block_counts, last_block_valid,
                       last_block_valid_default, num_seqs, strides, nullptr, 0, nullptr, 0, out,
                       blocks_per_split, stream, true);
}

pda_status pda_decode_masked(const pda_dims *dims, const void *q, const void *k_pool,
                             const void *v_pool, const int32_t *block_tables,
                             const int32_t *block_counts, const int32_t *last_block_valid,
                             int32_t last_block_valid_default, int32_t num_seqs,
                             pda_strides strides, const uint8_t *kv_mask, int64_t mask_stride,
                             void *workspace, size_t workspace_bytes, void *out,
                             int32_t blocks_per_split, void *stream) {
    clear_err();
    if (!kv_mask) return fail(PDA_ERR_NULL, "kv_mask is NULL");
    if (mask_stride < 1) return fail(PDA_ERR_DIMS, "mask_stride must be >= 1");
    return decode_impl(dims, q, k_pool, v_pool, block_tables, block_counts, last_block_valid,
                       last_block_valid_default, num_seqs, strides, kv_mask, mask_stride, workspace,
                       workspace_bytes, out, blocks_per_split, stream);
}

namespace {

constexpr int32_t kPrefillMinSplitTokens = 256;

int padded_dim(int D) { return D <= 64 ? 64 : (D <= 128 ? 128 : 256); }

// Pages per prefill split: the request clamped to [1, tile_capacity]; else
// whole page lists when the (sequence, kv head, row tile) items already give
// every SIMD a wave, otherwise about enough splits to do so, each of at
// least kPrefillMinSplitTokens tokens.
int32_t prefill_bps(const pda_dims *d, int32_t request, int64_t items, int cus) {
    const int32_t cap = d->tile_capacity;
    if (request > 0) return request > cap ? cap : request;
    const int64_t want = 4LL * cus;
    const int32_t min_bps = (int32_t)ceil_div(kPrefillMinSplitTokens, d->block_size);
    if (items >= want || min_bps >= cap) return cap;
    const int64_t nsp = ceil_div(want, items);
    int32_t bps = (int32_t)ceil_div(cap, nsp);
    if (bps < min_bps) bps = min_bps;
    return bps > cap ? cap : bps;
}

int32_t prefill_nsplit(const pda_dims *d, int32_t bps) { return (int32_t)ceil_div(d->tile_capacity, bps); }

size_t prefill_workspace_for(const pda_dims *d, int32_t q_len, int32_t bps) {
    const int32_t ns = prefill_nsplit(d, bps);
    if (ns <= 1) return 0;
    // (m, l) pairs, padded to 16 bytes, then the o rows
    return (size_t)d->max_seqs * q_len * d->num_q_heads * ns * (d->head_dim + 2) * sizeof(float) + 16;
}

}  // namespace

size_t pda_prefill_workspace_bytes(const pda_dims *d, int32_t q_len, int32_t request) {
    if (check_dims(d) != PDA_OK || q_len < 1) return 0;
    const int32_t min_bps = (int32_t)ceil_div(kPrefillMinSplitTokens, d->block_size);
    int32_t bps = request > 0 ? request : min_bps;
    if (bps > d->tile_capacity) bps = d->tile_capacity;
    return prefill_workspace_for(d, q_len, bps);
}

pda_status pda_prefill(const pda_dims *dims, int32_t q_len, const void *q, const void *k_pool,
                       const void *v_pool, const int32_t *block_tables,
                       const int32_t *block_counts, const int32_t *last_block_valid,
                       int32_t last_block_valid_default, int32_t num_seqs, pda_strides strides,
                       int32_t causal, const uint8_t *kv_mask, int64_t mask_seq_stride,
                       int64_t mask_q_stride, void *workspace, size_t workspace_bytes, void *out,
                       int32_t blocks_per_split, int32_t rows_per_wave, void *stream) {
    clear_err();
    pda_status st = check_dims(dims);
    if (st != PDA_OK) return st;
    if (num_seqs < 0 || num_seqs > dims->max_seqs)
        return fail(PDA_ERR_MAX_SEQS, "num_seqs %d outside [0, max_seqs=%d]", num_seqs, dims->max_seqs);
    const int G = dims->num_q_heads / dims->num_kv_heads;
    if (q_len < 1 || (int64_t)q_len * G > (int64_t(1) << 24))
        return fail(PDA_ERR_DIMS, "q_len %d outside [1, 2^24 / gqa_ratio]", q_len);
    if (blocks_per_split < 0) return fail(PDA_ERR_DIMS, "blocks_per_split must be >= 0");
    if (rows_per_wave != 0 && rows_per_wave != 16 && rows_per_wave != 32 && rows_per_wave != 64)
        return fail(PDA_ERR_DIMS, "rows_per_wave must be 0, 16, 32 or 64");
    if ((st = check_tile_ptrs(q, k_pool, v_pool, block_tables, block_counts, last_block_valid)) != PDA_OK)
        return st;
    if (!out) return fail(PDA_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(PDA_ERR_ALIGN, "out must be 16-byte aligned");
    if ((st = check_strides(dims, strides)) != PDA_OK) return st;
    if (kv_mask && (mask_seq_stride < 0 || mask_q_stride < 0))
        return fail(PDA_ERR_DIMS, "mask strides must be >= 0");
    if (workspace && !aligned(workspace, 16))
        return fail(PDA_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (num_seqs == 0) return PDA_OK;

    const int dp = padded_dim(dims->head_dim);
    int rb = rows_per_wave / 16;
    const int max_rb = pda::prefill_max_rb(dp, kv_mask != nullptr);
    const int cus = device_cus();
    if (rb == 0) {   // 16 rows per wave when they cover a kv head's rows, else 32: at 32
                     // rows two waves fit each SIMD (64 rows are left to explicit requests)
        const int64_t rows = (int64_t)q_len * G;
        rb = rows <= 16 ? 1 : 2;
        if (rb == 2 && dp <= 128) {
            // ... and 16 when the tile groups of 32-row waves fit one round of
            // the resident workgroups (two per CU) and the work is causal or
            // would still fit it at 16: twice the tile groups, and for causal
            // work two laps that pair the triangle's long tile groups with its
            // short ones (measured on MI355X: one 2048-token causal prompt,
            // 32/8 heads, 74.7 -> 69.1 us)
            const int64_t t2 = ceil_div(rows, 32);
            const int64_t items2 = (int64_t)num_seqs * dims->num_kv_heads * t2;
            const int32_t ns2 = prefill_nsplit(dims, prefill_bps(dims, blocks_per_split, items2, cus));
            const int64_t need2 = ceil_div((int64_t)num_seqs * ns2 * dims->num_kv_heads, 8) * ceil_div(t2, 4);
            const int64_t resident = (int64_t)(cus >= 8 ? cus / 8 : 1) * 2;   // workgroups per XCD
            if (need2 <= resident && (causal || 2 * need2 <= resident)) rb = 1;
        }
    }
    if (rb > max_rb) rb = max_rb;
    const int32_t ntiles = (int32_t)ceil_div((int64_t)q_len * G, 16 * rb);
    const int64_t items = (int64_t)num_seqs * dims->num_kv_heads * ntiles;
    const int32_t bps = prefill_bps(dims, blocks_per_split, items, cus);
    const int32_t nsplit = prefill_nsplit(dims, bps);
    if ((int64_t)num_seqs * nsplit * dims->num_kv_heads * ntiles > (int64_t(1) << 31) - 4096)
        return fail(PDA_ERR_DIMS, "too many work items");
    const size_t need = prefill_workspace_for(dims, q_len, bps);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PDA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);

    pda::PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k_pool);
    a.v = static_cast<const uint16_t *>(v_pool);
    a.blocks = block_tables;
    a.counts = block_counts;
    a.lastv = last_block_valid;
    a.mask = kv_mask;
    a.mask_ss = kv_mask ? mask_seq_stride : 0;
    a.mask_qs = kv_mask ? mask_q_stride : 0;
    a.out = static_cast<uint16_t *>(out);
    a.part_ml = static_cast<float *>(workspace);
    const int64_t ml_floats = ((int64_t)num_seqs * q_len * dims->num_q_heads * nsplit * 2 + 3) / 4 * 4;
    a.part_o = a.part_ml ? a.part_ml + ml_floats : nullptr;
    a.blk = strides.blk;
    a.tok = strides.tok;
    a.kvh = strides.kvh;
    a.bs_magic = ((uint64_t(1) << 32) + (uint64_t)dims->block_size - 1) / (uint64_t)dims->block_size;
    a.S = num_seqs;
    a.Q = q_len;
    a.Hq = dims->num_q_heads;
    a.Hkv = dims->num_kv_heads;
    a.G = G;
    a.D = dims->head_dim;
    a.bs = dims->block_size;
    a.cap = dims->tile_capacity;
    a.lv_default = last_block_valid_default;
    a.span = bps * dims->block_size;
    a.nsplit = nsplit;
    a.ntiles = ntiles;
    a.causal = causal ? 1 : 0;
    a.cus = cus;
    a.longest_first = 0;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dims->head_dim));
    hipError_t e = pda::launch_prefill(a, dp, rb, static_cast<hipStream_t>(stream), take_events());
    return e == hipSuccess ? PDA_OK : hip_fail(e, "prefill launch");
}

namespace {

pda_status check_rope_common(const void *x, const float *cos_table, const float *sin_table,
                             const int32_t *positions, int64_t num_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t max_positions) {
    if (!x || !cos_table || !sin_table || !positions)
        return fail(PDA_ERR_NULL, "a required pointer is NULL");
    if (num_tokens < 0 || num_heads < 1 || max_positions < 1)
        return fail(PDA_ERR_DIMS, "num_tokens >= 0, num_heads >= 1 and max_positions >= 1 required");
    if (head_dim < 8 || head_dim > 256 || head_dim % 8 != 0)
        return fail(PDA_ERR_HEAD_DIM, "head_dim %d must be a multiple of 8 in [8, 256]", head_dim);
    if (!aligned(x, 16) || !aligned(cos_table, 16) || !aligned(sin_table, 16))
        return fail(PDA_ERR_ALIGN, "rows and cos/sin tables must be 16-byte aligned");
    if (!aligned(positions, 4)) return fail(PDA_ERR_ALIGN, "positions must be 4-byte aligned");
    if (num_tokens > (int64_t(1) << 40) / ((int64_t)num_heads * head_dim))
        return fail(PDA_ERR_DIMS, "too many elements");
    return PDA_OK;
}

}  // namespace

pda_status pda_rope(const void *x, void *out, int64_t num_tokens, int32_t num_heads,
                    int32_t head_dim, const float *cos_table, const float *sin_table,
                    int32_t max_positions, const int32_t *positions, void *stream) {
    clear_err();
    pda_status st = check_rope_common(x, cos_table, sin_table, positions, num_tokens, num_heads,
                                      head_dim, max_positions);
    if (st != PDA_OK) return st;
    if (!out) return fail(PDA_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(PDA_ERR_ALIGN, "out must be 16-byte aligned");
    if (num_tokens == 0) return PDA_OK;
    pda::RopeArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.out = static_cast<uint16_t *>(out);
    a.cos_t = cos_table;
    a.sin_t = sin_table;
    a.positions = positions;
    a.T = num_tokens;
    a.H = num_heads;
    a.D = head_dim;
    a.max_pos = max_positions;
    hipError_t e = pda::launch_rope(a, device_cus(), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PDA_OK : hip_fail(e, "rope launch");
}

pda_status pda_rope_append_kv(const pda_dims *dims, const void *k_new, const void *v_new,
                              int64_t num_tokens, const int32_t *token_seq,
                              const int32_t *positions, const float *cos_table,
                              const float *sin_table, int32_t max_positions,
                              const int32_t *block_tables, void *k_pool, void *v_pool,
                              pda_strides strides, void *stream) {
    clear_err();
    pda_status st = check_dims(dims);
    if (st != PDA_OK) return st;
    if ((st = check_rope_common(k_new, cos_table, sin_table, positions, num_tokens,
                                dims->num_kv_heads, dims->head_dim, max_positions)) != PDA_OK)
        return st;
    if (!v_new || !token_seq || !block_tables || !k_pool || !v_pool)
        return fail(PDA_ERR_NULL, "a required pointer is NULL");
    if (!aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
        return fail(PDA_ERR_ALIGN, "v_new and the pools must be 16-byte aligned");
    if (!aligned(token_seq, 4) || !aligned(block_tables, 4))
        return fail(PDA_ERR_ALIGN, "token_seq and block_tables must be 4-byte aligned");
    if ((st = check_strides(dims, strides)) != PDA_OK) return st;
    if (num_tokens == 0) return PDA_OK;
    pda::RopeArgs a{};
    a.x = static_cast<const uint16_t *>(k_new);
    a.v_new = static_cast<const uint16_t *>(v_new);
    a.k_pool = static_cast<uint16_t *>(k_pool);
    a.v_pool = static_cast<uint16_t *>(v_pool);
    a.cos_t = cos_table;
    a.sin_t = sin_table;
    a.positions = positions;
    a.token_seq = token_seq;
    a.blocks = block_tables;
    a.T = num_tokens;
    a.blk = strides.blk;
    a.tok = strides.tok;
    a.kvh = strides.kvh;
    a.H = dims->num_kv_heads;
    a.D = dims->head_dim;
    a.max_pos = max_positions;
    a.S = dims->max_seqs;
    a.cap = dims->tile_capacity;
    a.bs = dims->block_size;
    hipError_t e = pda::launch_rope_append_kv(a, device_cus(), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PDA_OK : hip_fail(e, "rope append launch");
}

pda_status pda_debug_time_attention(void *before, void *after) {
    clear_err();
    if ((before == nullptr) != (after == nullptr))
        return fail(PDA_ERR_NULL, "both events or neither must be given");
    t_events.before = static_cast<hipEvent_t>(before);
    t_events.after = static_cast<hipEvent_t>(after);
    return PDA_OK;
}

const char *pda_status_string(pda_status status) {
    // a C caller may pass any int: read it as one rather than as the enum
    int s = 0;
    static_assert(sizeof(status) == sizeof(s), "pda_status is int-sized");
    memcpy(&s, &status, sizeof s);
    switch (s) {
        case PDA_OK: return "PDA_OK";
        case PDA_ERR_NULL: return "PDA_ERR_NULL";
        case PDA_ERR_DIMS: return "PDA_ERR_DIMS";
        case PDA_ERR_GQA: return "PDA_ERR_GQA";
        case PDA_ERR_HEAD_DIM: return "PDA_ERR_HEAD_DIM";
        case PDA_ERR_MAX_SEQS: return "PDA_ERR_MAX_SEQS";
        case PDA_ERR_ALIGN: return "PDA_ERR_ALIGN";
        case PDA_ERR_WORKSPACE: return "PDA_ERR_WORKSPACE";
        case PDA_ERR_HIP: return "PDA_ERR_HIP";
    }
    return "PDA_ERR_UNKNOWN";
}

const char *pda_last_error(void) { return g_err; }

}  // extern "C"
