// Host half of libddp: bucket planning, the per-iteration reducer state
// machine and the launcher that feeds the bucket reduction kernels.
//
// Sources are cited by tag and section; the tags are defined in include/ddp.h.
#include "../../include/ddp.h"
#include "internal.h"
#include "static_area.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <limits>
#include <memory>
#include <new>
#include <string>
#include <vector>

using ddp::DeviceSeg;
using ddp::KernelTables;

namespace {

// Text of the last error on this thread. Recording it never throws: when
// the text cannot be stored (out of host memory), g_err_fixed points to a
// static text instead.
thread_local std::string g_err;
thread_local const char *g_err_fixed = nullptr;
constexpr const char *kNoMemText = "out of host memory";

int fail(int code, const std::string &msg) noexcept
{
    try {
        g_err.assign(msg);
        g_err_fixed = nullptr;
    } catch (...) {
        g_err_fixed = kNoMemText;
    }
    return code;
}

int fail(int code, const char *msg) noexcept
{
    try {
        g_err.assign(msg);
        g_err_fixed = nullptr;
    } catch (...) {
        g_err_fixed = kNoMemText;
    }
    return code;
}

int hip_fail(const char *what, hipError_t e) noexcept
{
    try {
        g_err.assign(what);
        g_err.append(": ");
        g_err.append(hipGetErrorString(e));
        g_err_fixed = nullptr;
    } catch (...) {
        g_err_fixed = kNoMemText;
    }
    return DDP_ERR_HIP;
}

// *captured: whether work enqueued on s is being recorded into a HIP graph
// (stream capture) rather than run. The null stream cannot be captured.
hipError_t is_captured(hipStream_t s, bool *captured) noexcept
{
    *captured = false;
    if (!s) return hipSuccess;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(s, &st);
    *captured = e == hipSuccess && st != hipStreamCaptureStatusNone;
    return e;
}

// Every entry point runs its body through this: the C ABI never lets an
// exception out. Host memory exhaustion (std::bad_alloc from a container or
// a message) becomes DDP_ERR_NOMEM; anything else DDP_ERR_INVALID.
template <class F>
int guarded(F &&body) noexcept
{
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return fail(DDP_ERR_NOMEM, kNoMemText);
    } catch (...) {
        return fail(DDP_ERR_INVALID, "internal error: unexpected exception in the host library");
    }
}

std::string list_params(const std::vector<int32_t> &ps)
{
    std::string s;
    size_t shown = 0;
    for (int32_t p : ps) {
        if (shown == 64) {
            s += " ... (" + std::to_string(ps.size()) + " in all)";
            break;
        }
        s += (shown ? " " : "") + std::to_string(p);
        ++shown;
    }
    return s;
}

// Workgroups of one launch resident per CU (0: as many as registers allow).
// The kernel uses no LDS; the launch reserves LDS only so that the hardware
// dispatcher keeps at most this many workgroups on a CU. Fewer tiles in
// flight keep each of the 2W streams' in-flight window narrow (a few MiB
// across the chip), which measured 2-8% faster than full occupancy for
// W >= 3: one per CU with the larger tiles (U = 4 for fp32 gradients, U = 2
// for bf16 wgrads at W = 16), two with the small ones (U = 1) and for the
// reduce-scatter. W <= 2 (four streams), and the all-reduce of bf16 wgrads
// into fp32 main_grad at W = 3, 4 (never measured capped), run at full
// occupancy. So does W > 32: the generic kernel loads eight replicas per
// round trip and needs every resident workgroup to hide the latency
// (capped at two per CU it ran a third slower).
// bf16_accum: input mode DDP_IN_BF16_ACCUM_F32.
constexpr int auto_workgroups_per_cu(int W, bool reduce_scatter, bool bf16_accum)
{
    if (W <= 2 || W > 32) return 0;
    if (reduce_scatter) return 2;
    if (ddp::unroll_for(W, false, bf16_accum) == 1) return 2;
    return bf16_accum && W <= 4 ? 0 : 1;
}

constexpr size_t kAlign = 256;

// Event pairs in a reducer's timing ring (its only HIP events besides the
// three stream-ordering ones and the two staging ones).
constexpr int kTimingSlots = 256;

size_t align_up(size_t x)
{
    return (x + kAlign - 1) / kAlign * kAlign;
}

// Plan data validated and normalised from a desc.
struct PlanView {
    int32_t W = 0, P = 0, B = 0, mode = 0;
    bool reduce_scatter = false;
    bool find_unused = false;
    std::vector<int64_t> numel;
    std::vector<int32_t> bucket_of;
    std::vector<int64_t> offset;                 // bytes inside the bucket
    std::vector<std::vector<int32_t>> members;   // flat-buffer order
    std::vector<int64_t> bucket_bytes, bucket_flat;
    // device tables (built only when buffers are given)
    std::vector<DeviceSeg> segs;
    std::vector<int32_t> tile_seg;
    std::vector<int32_t> tile_begin, tile_count;
};

// Segments of every bucket: runs inside one gradient and one ring chunk. The
// chunk of bucket element e is e / q with q = ceil(n / W) [DDP-ch17 §17.4].
int build_segments(PlanView &pv, bool split_by_param)
{
    const int64_t TILE = ddp::tile_elems(pv.W, pv.reduce_scatter, pv.mode == DDP_IN_BF16_ACCUM_F32);
    pv.segs.clear();
    pv.tile_seg.clear();
    pv.tile_begin.assign(pv.B, 0);
    pv.tile_count.assign(pv.B, 0);
    int64_t tiles = 0;
    auto add = [&](int b, int64_t flat, int64_t src, int64_t len, int32_t param, int32_t chunk) -> bool {
        if (len <= 0) return true;
        DeviceSeg s{};
        s.flat = flat;
        s.src = src;
        s.len = len;
        s.param = param;
        s.chunk = chunk;
        s.tile0 = int32_t(tiles);
        s.head = -1;
        s.used = ~uint64_t(0);
        int64_t nt = (len + TILE - 1) / TILE;
        if (tiles + nt > std::numeric_limits<int32_t>::max()) return false;
        int32_t id = int32_t(pv.segs.size());
        pv.segs.push_back(s);
        for (int64_t t = 0; t < nt; ++t) pv.tile_seg.push_back(id);
        tiles += nt;
        pv.tile_count[b] += int32_t(nt);
        return true;
    };
    for (int b = 0; b < pv.B; ++b) {
        pv.tile_begin[b] = int32_t(tiles);
        const int64_t n = pv.bucket_bytes[b] / 4;
        const int64_t base = pv.bucket_flat[b] / 4;
        if (n == 0) continue;
        const int64_t q = (n + pv.W - 1) / pv.W;
        if (!split_by_param) {
            for (int c = 0; c < pv.W; ++c) {
                int64_t lo = std::min(n, int64_t(c) * q), hi = std::min(n, int64_t(c + 1) * q);
                if (!add(b, base + lo, 0, hi - lo, -1, c)) return fail(DDP_ERR_INVALID, "too many tiles");
            }
            continue;
        }
        for (int32_t p : pv.members[b]) {
            const int64_t a = pv.offset[p] / 4, len = pv.numel[p];
            int64_t i = 0;
            while (i < len) {
                const int64_t e = a + i;
                const int32_t c = int32_t(e / q);
                const int64_t run = std::min(len - i, int64_t(c + 1) * q - e);
                if (!add(b, base + e, i, run, p, c)) return fail(DDP_ERR_INVALID, "too many tiles");
                i += run;
            }
        }
    }
    return DDP_OK;
}

int validate(const ddp_reducer_desc *d, PlanView &pv)
{
    if (!d) return fail(DDP_ERR_INVALID, "desc is NULL");
    if (d->world < 1 || d->world > 1024) return fail(DDP_ERR_INVALID, "world must be in [1, 1024]");
    if (d->n_params < 0 || d->n_buckets < 0) return fail(DDP_ERR_INVALID, "negative parameter or bucket count");
    if (d->input_mode < DDP_IN_F32_COPY || d->input_mode > DDP_IN_BF16_ACCUM_F32)
        return fail(DDP_ERR_INVALID, "unknown input mode");
    if (d->collective != DDP_ALL_REDUCE && d->collective != DDP_REDUCE_SCATTER)
        return fail(DDP_ERR_INVALID, "unknown collective");
    if (d->find_unused && d->world > 64)
        return fail(DDP_ERR_INVALID, "unused-parameter detection supports at most 64 replicas");
    if (d->n_params > 0 && (!d->param_numel || !d->bucket_of || !d->offset_in_bucket))
        return fail(DDP_ERR_INVALID, "plan arrays are NULL");
    pv.W = d->world;
    pv.P = d->n_params;
    pv.B = d->n_buckets;
    pv.mode = d->input_mode;
    pv.reduce_scatter = d->collective == DDP_REDUCE_SCATTER;
    pv.find_unused = d->find_unused != 0;
    pv.numel.assign(d->param_numel, d->param_numel + pv.P);
    pv.bucket_of.assign(d->bucket_of, d->bucket_of + pv.P);
    pv.offset.assign(d->offset_in_bucket, d->offset_in_bucket + pv.P);
    pv.members.assign(pv.B, {});
    for (int32_t p = 0; p < pv.P; ++p) {
        if (pv.numel[p] < 0 || pv.numel[p] > (std::numeric_limits<int64_t>::max() >> 3))
            return fail(DDP_ERR_INVALID, "gradient " + std::to_string(p) + " has a bad size");
        if (pv.bucket_of[p] < 0 || pv.bucket_of[p] >= pv.B)
            return fail(DDP_ERR_INVALID, "gradient " + std::to_string(p) + " has no valid bucket");
        if (pv.offset[p] < 0 || pv.offset[p] % 4)
            return fail(DDP_ERR_INVALID, "gradient " + std::to_string(p) + " has a bad offset");
        pv.members[pv.bucket_of[p]].push_back(p);
    }
    pv.bucket_bytes.assign(pv.B, 0);
    pv.bucket_flat.assign(pv.B, 0);
    int64_t running = 0;
    for (int b = 0; b < pv.B; ++b) {
        auto &m = pv.members[b];
        if (m.empty()) return fail(DDP_ERR_INVALID, "bucket " + std::to_string(b) + " holds no gradient");
        std::stable_sort(m.begin(), m.end(), [&](int32_t x, int32_t y) {
            return pv.offset[x] != pv.offset[y] ? pv.offset[x] < pv.offset[y] : pv.numel[x] < pv.numel[y];
        });
        int64_t off = 0;
        for (int32_t p : m) {
            if (pv.offset[p] != off)
                return fail(DDP_ERR_INVALID, "bucket " + std::to_string(b) + ": gradients do not tile the bucket");
            if (pv.numel[p] > (std::numeric_limits<int64_t>::max() - off) / 4)
                return fail(DDP_ERR_INVALID, "bucket " + std::to_string(b) + " exceeds 2^63 bytes");
            off += 4 * pv.numel[p];
        }
        if (off > std::numeric_limits<int64_t>::max() - running)
            return fail(DDP_ERR_INVALID, "flat buffer exceeds 2^63 bytes");
        pv.bucket_bytes[b] = off;
        pv.bucket_flat[b] = running;
        running += off;
    }
    return DDP_OK;
}

struct Layout {
    size_t grads_off = 0, flat_off = 0, segs_off = 0, tiles_off = 0, total = 0;
};

Layout layout_of(const PlanView &pv)
{
    Layout l;
    size_t cur = 0;
    l.grads_off = cur;
    if (pv.mode != DDP_IN_F32_VIEW) cur = align_up(cur + sizeof(void *) * size_t(pv.W) * size_t(pv.P));
    l.flat_off = cur;
    cur = align_up(cur + sizeof(float *) * size_t(pv.W));
    l.segs_off = cur;
    cur = align_up(cur + sizeof(DeviceSeg) * pv.segs.size());
    l.tiles_off = cur;
    cur = align_up(cur + sizeof(int32_t) * pv.tile_seg.size());
    l.total = cur;
    return l;
}

}  // namespace

struct ddp_reducer {
    PlanView pv;
    bool device = false;
    ddp::Scale scale{1.0f, 1.0f, 0};
    int32_t builtin_hook = DDP_HOOK_ALLREDUCE;   // kernel family of every launch
    int32_t workgroups_per_cu = 0;               // 0: automatic, < 0: no cap, 1..8: cap
    int lds_per_cu = 0, lds_per_block = 0;       // the device's LDS sizes (bytes)

    // set while a launch is issued beside a running backward (see
    // issue_buckets)
    bool beside_backward = false;

    // Workgroups of the next launch resident per CU (0: no cap). Beside a
    // running backward the automatic rule allows one workgroup per CU, which
    // leaves the backward's kernels most of each CU's LDS and wave slots; the
    // exposed tail gets the rule tuned for bandwidth.
    int launch_k() const
    {
        int k = workgroups_per_cu == 0 ? auto_workgroups_per_cu(pv.W, pv.reduce_scatter,
                                                                 pv.mode == DDP_IN_BF16_ACCUM_F32)
                                       : (workgroups_per_cu < 0 ? 0 : workgroups_per_cu);
        if (workgroups_per_cu == 0 && beside_backward && k > 1) k = 1;
        return k;
    }
    // LDS each launch reserves so that at most k of its workgroups share a CU.
    unsigned launch_lds() const
    {
        const int k = launch_k();
        if (k <= 0 || lds_per_cu <= 0) return 0;
        int bytes = lds_per_cu / (k + 1) + 2048;   // k fit, k + 1 do not
        bytes = (bytes + 255) / 256 * 256;
        return unsigned(std::min(bytes, lds_per_block));
    }
    // At one workgroup per CU the small-tile instances (W = 5..8 all-reduce)
    // give each workgroup two tiles, so that a CU keeps the bytes in flight
    // of the two workgroups their tuned rule allows.
    bool launch_pair() const
    {
        return launch_k() == 1 && lds_per_cu > 0 &&
               ddp::pairs_tiles(pv.W, pv.reduce_scatter, false, pv.mode == DDP_IN_BF16_ACCUM_F32);
    }
    KernelTables tables{};
    // tables in the static area of this device (ddp_reducer_create_static),
    // valid while the area's generation is the one this reducer claimed
    int static_device = -1;
    uint64_t static_generation = 0;
    hipStream_t compute = nullptr, comm = nullptr;
    // ev_ready: compute -> comm before a launch; ev_done: comm -> compute at
    // finish (device-scope release suffices between two streams of one
    // device); ev_host (system scope): what a host-blocking finish waits on.
    // ev_ready keeps the default system-scope release: with device scope the
    // HIP runtime made every launch of a many-launch step about 20 us slower.
    hipEvent_t ev_ready = nullptr, ev_done = nullptr, ev_host = nullptr;
    // unused detection: ev_tables orders a reduction on another stream after
    // the segment-table upload on the comm stream; ev_foreign orders later
    // uploads after that reduction
    hipEvent_t ev_tables = nullptr, ev_foreign = nullptr;
    // per-launch timing: a fixed ring of event pairs. Record i uses pair
    // i mod kTimingSlots; before a pair is recorded again, the launch that
    // last used it is waited for and its duration copied to the host record.
    bool timing = false;
    struct TimingRec {
        int32_t first, count;   // first bucket of the launch, buckets it covered
        float ms;               // kernel duration; read from the events once resolved
    };
    mutable std::vector<TimingRec> timed;   // launches since timing was last enabled
    mutable size_t timed_resolved = 0;      // records [0, timed_resolved) hold their ms
    hipEvent_t ring0[kTimingSlots] = {}, ring1[kTimingSlots] = {};
    ddp_comm_hook_fn hook = nullptr;
    void *hook_ctx = nullptr;
    // unused-parameter detection and no_sync [DDP-ch17 §17.33; PTD-notes §2.2.3, §2.2.4]
    bool require_sync = true;             // read at the next prepare
    bool sync = true;                     // this backward reduces
    std::vector<uint8_t> window;          // [W*P] OR of the used tables since the last synchronized pass
    bool window_set = false;
    std::vector<uint64_t> masks;          // [P] bit w: replica w contributes gradient p
    bool masks_uploaded = false;
    DeviceSeg *stage = nullptr;           // pinned host staging, 2 slots of the segment table
    hipEvent_t stage_ev[2] = {nullptr, nullptr};
    int stage_slot = 0;
    DeviceSeg *segs_dev = nullptr;        // the segment table inside the workspace
    std::vector<uint64_t> device_masks;   // [P] the masks that table holds (its last upload)

    // the segment table with each segment's mask (its gradient's); with
    // unused detection every segment lies inside one gradient
    void segment_records(DeviceSeg *out) const
    {
        for (size_t i = 0; i < pv.segs.size(); ++i) {
            out[i] = pv.segs[i];
            out[i].used = masks[size_t(pv.segs[i].param)];
        }
    }
    // per-iteration state [DDP-ch17 §17.12, §17.16]
    std::vector<int32_t> pending;
    // bucket groups [MegatronDDP §3]: group g = buckets [group_first[g],
    // group_first[g + 1]), issued as one launch once all of them are ready
    std::vector<int32_t> group_first;     // [G + 1], last entry B
    std::vector<int32_t> group_of;        // [B]
    std::vector<int32_t> group_pending;   // [G] gradients the group still waits for
    std::vector<uint8_t> ready;
    std::vector<int32_t> ready_order;
    int32_t next = 0;
    int64_t marks = 0;
    bool finished = false;
    // a launch of this backward failed (hook error or HIP error): buckets from
    // failed_bucket on were not reduced and nothing more launches until reset
    int32_t failed_bucket = -1;
    int failed_code = DDP_OK;
    std::string failed_msg;

    void reset()
    {
        failed_bucket = -1;
        failed_code = DDP_OK;
        failed_msg.clear();
        masks_uploaded = false;
        pending.resize(pv.B);
        for (int b = 0; b < pv.B; ++b) pending[b] = int32_t(pv.members[b].size());
        count_groups();
        ready.assign(pv.P, 0);
        ready_order.clear();
        next = 0;
        marks = 0;
        finished = false;
    }
    std::vector<int32_t> unready() const
    {
        std::vector<int32_t> out;
        for (int32_t p = 0; p < pv.P; ++p)
            if (!ready[p]) out.push_back(p);
        return out;
    }
    // a synchronized backward has started and neither finished nor failed
    bool in_iteration() const { return sync && marks > 0 && !finished && failed_bucket < 0; }

    // the end of a synchronized backward: the next window of used tables starts empty
    void end_window()
    {
        if (!pv.find_unused) return;
        std::fill(window.begin(), window.end(), 0);
        window_set = false;
    }

    // builds the new group tables aside and swaps them in, so an allocation
    // failure leaves the old grouping in place
    void set_groups(const int32_t *first, int32_t n)
    {
        std::vector<int32_t> gf, go(size_t(pv.B)), gp;
        if (first)
            gf.assign(first, first + n);
        else
            for (int32_t b = 0; b < pv.B; ++b) gf.push_back(b);
        gf.push_back(pv.B);
        for (size_t g = 0; g + 1 < gf.size(); ++g)
            for (int32_t b = gf[g]; b < gf[g + 1]; ++b) go[b] = int32_t(g);
        gp.assign(gf.size() - 1, 0);
        for (int b = 0; b < pv.B; ++b) gp[go[b]] += pending.empty() ? 0 : pending[b];
        group_first.swap(gf);
        group_of.swap(go);
        group_pending.swap(gp);
    }

    void count_groups()
    {
        std::fill(group_pending.begin(), group_pending.end(), 0);
        for (int b = 0; b < pv.B; ++b) group_pending[group_of[b]] += pending[b];
    }

    // moves next past every group that is complete, in order
    void advance()
    {
        while (next < pv.B && group_pending[group_of[next]] == 0) next = group_first[group_of[next] + 1];
    }

    // the per-gradient replica masks of this synchronization window
    void compute_masks()
    {
        const uint64_t all = pv.W >= 64 ? ~uint64_t(0) : ((uint64_t(1) << pv.W) - 1);
        masks.assign(pv.P, window_set ? 0 : all);
        if (!window_set) return;
        // replica-major rows, one contiguous pass each (window entries are 0 or 1)
        uint64_t *m = masks.data();
        const int W = pv.W;
        const int32_t P = pv.P;
        for (int w = 0; w < W; ++w) {
            const uint8_t *row = window.data() + size_t(w) * P;
            for (int32_t p = 0; p < P; ++p) m[p] |= uint64_t(row[p]) << w;
        }
    }
};

namespace {

// Copies the durations of timing records [r->timed_resolved, upto) from
// their event pairs to the host records, waiting for those launches.
int resolve_timings(const ddp_reducer *r, size_t upto)
{
    for (size_t i = r->timed_resolved; i < upto; ++i) {
        const size_t slot = i % kTimingSlots;
        hipError_t e = hipEventSynchronize(r->ring1[slot]);
        if (e == hipSuccess) e = hipEventElapsedTime(&r->timed[i].ms, r->ring0[slot], r->ring1[slot]);
        if (e != hipSuccess) return hip_fail("reading a launch's timing events", e);
        r->timed_resolved = i + 1;
    }
    return DDP_OK;
}

// Reduction of buckets [b0, b1) (consecutive, so their tiles are one
// contiguous range of the tile table) as one kernel launch on stream s.
// With timing on, the launch is bracketed by the next event pair of the
// ring; a pair still holding an unread launch is read first (waiting for
// that launch, kTimingSlots launches back).
int enqueue_reduce(ddp_reducer *r, int32_t b0, int32_t b1, hipStream_t s)
{
    if (!r->device) return fail(DDP_ERR_INVALID, "reducer has no device buffers");
    if (r->static_generation && ddp::static_table_generation(r->static_device) != r->static_generation)
        return fail(DDP_ERR_INVALID, "this reducer's tables in the static table area of device " +
                                         std::to_string(r->static_device) +
                                         " were replaced by a later ddp_reducer_create_static");
    hipError_t e;
    const size_t rec = r->timed.size();
    const size_t slot = rec % kTimingSlots;
    if (r->timing) {
        bool captured = false;
        if ((e = is_captured(s, &captured)) != hipSuccess) return hip_fail("stream capture status", e);
        if (captured)
            return fail(DDP_ERR_INVALID, "per-launch timing reads its events on the host: it is not available "
                                         "while the stream is captured into a graph");
        if (rec >= kTimingSlots) {
            const int rc = resolve_timings(r, rec - kTimingSlots + 1);
            if (rc != DDP_OK) return rc;
        }
        if (!r->ring0[slot]) {
            e = hipEventCreateWithFlags(&r->ring0[slot], hipEventDisableSystemFence);
            if (e != hipSuccess) {
                r->ring0[slot] = nullptr;
                return hip_fail("hipEventCreate", e);
            }
        }
        if (!r->ring1[slot]) {
            e = hipEventCreateWithFlags(&r->ring1[slot], hipEventDisableSystemFence);
            if (e != hipSuccess) {
                r->ring1[slot] = nullptr;
                return hip_fail("hipEventCreate", e);
            }
        }
        r->timed.push_back({b0, b1 - b0, 0.0f});   // may throw: nothing is enqueued yet
        if ((e = hipEventRecord(r->ring0[slot], s)) != hipSuccess) {
            r->timed.pop_back();
            return hip_fail("hipEventRecord", e);
        }
    }
    const int32_t tile0 = r->pv.tile_begin[b0];
    const int32_t tiles = r->pv.tile_begin[b1 - 1] + r->pv.tile_count[b1 - 1] - tile0;
    const unsigned lds = r->launch_lds();
    const bool pair = r->launch_pair();
    const PlanView &pv = r->pv;
    switch (r->builtin_hook) {
    case DDP_HOOK_BF16_COMPRESS:
        e = ddp::launch_bf16_hook(pv.mode, pv.W, pv.reduce_scatter, r->scale, r->tables, tile0, tiles, lds, pair, s);
        break;
    case DDP_HOOK_FP16_COMPRESS:
        e = ddp::launch_fp16_hook(pv.mode, pv.W, pv.reduce_scatter, r->scale, r->tables, tile0, tiles, lds, pair, s);
        break;
    default:
        e = ddp::launch_mean(pv.mode, pv.W, pv.reduce_scatter, r->scale, r->tables, tile0, tiles, lds, pair, s);
        break;
    }
    if (e != hipSuccess) {
        if (r->timing) r->timed.pop_back();
        return hip_fail("bucket reduce launch", e);
    }
    if (r->timing && (e = hipEventRecord(r->ring1[slot], s)) != hipSuccess) {
        r->timed.pop_back();
        return hip_fail("hipEventRecord", e);
    }
    return DDP_OK;
}

// The replica masks of this backward go to the device once, on the comm
// stream, ahead of its first reduction: the per-replica "used" tables reduced
// over replicas (a bitwise OR) [DDP-ch17 §17.33; PTD-notes §3.2]. Masks equal
// to those of the last upload are not sent again.
int upload_masks(ddp_reducer *r)
{
    if (!r->pv.find_unused || !r->device || r->masks_uploaded || r->pv.segs.empty()) return DDP_OK;
    if (r->masks == r->device_masks) {   // the usual case: the same gradients unused as last time
        r->masks_uploaded = true;
        return DDP_OK;
    }
    const int slot = r->stage_slot;
    r->stage_slot ^= 1;
    hipError_t e = hipEventSynchronize(r->stage_ev[slot]);   // the copy that last used this slot is done
    if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
    const size_t n = r->pv.segs.size();
    DeviceSeg *h = r->stage + size_t(slot) * n;
    r->segment_records(h);
    r->device_masks.clear();   // unknown from here until the copy is queued: a failure forces a new upload
    e = hipMemcpyAsync(r->segs_dev, h, sizeof(DeviceSeg) * n, hipMemcpyHostToDevice, r->comm);
    if (e == hipSuccess) e = hipEventRecord(r->stage_ev[slot], r->comm);
    if (e != hipSuccess) return hip_fail("mask upload", e);
    r->device_masks = r->masks;
    r->masks_uploaded = true;
    return DDP_OK;
}

// All-reduce of buckets [b0, b1) as issued by the reducer: the comm stream
// first waits for everything queued on the compute stream (the buckets'
// gradients were produced there), then the hook runs once per bucket, in
// order, or the default reduction covers the whole range in one launch
// [PTD-notes §2.3; MegatronDDP §3]. When the compute stream has already
// drained, every gradient it produced is complete and visible, so the
// cross-stream event (a few microseconds of queue latency) is skipped.
// On failure *at is the first bucket not issued.
int issue_buckets(ddp_reducer *r, int32_t b0, int32_t b1, int32_t *at)
{
    *at = b0;
    // the occupancy rule for a launch beside a running backward applies to
    // this call's launches only
    struct Reset {
        ddp_reducer *r;
        ~Reset() { r->beside_backward = false; }
    } reset{r};
    bool captured = false;
    if (r->device) {
        const hipError_t e = is_captured(r->compute, &captured);
        if (e != hipSuccess) return hip_fail("stream capture status", e);
        // Checked before anything is enqueued, so a refused launch leaves the
        // capture as it was. Replays of a graph cannot change the replica
        // masks, which are host state of each backward, nor read timing
        // events on the host.
        if (captured && r->pv.find_unused)
            return fail(DDP_ERR_INVALID, "unused-parameter detection is not available while the compute stream "
                                         "is captured into a graph (the replica masks are host state)");
        if (captured && r->timing)
            return fail(DDP_ERR_INVALID, "per-launch timing reads its events on the host: it is not available "
                                         "while the compute stream is captured into a graph");
    }
    if (r->device && r->compute != r->comm) {
        // Under stream capture nothing has run and a stream query would break
        // the capture: the launch always waits, and the graph keeps that wait
        // as an edge from the compute stream's work to the reduction.
        hipError_t e = captured ? hipErrorNotReady : hipStreamQuery(r->compute);
        if (e == hipErrorNotReady) {
            // The compute stream has work queued. A launch that does not hold
            // the backward's last bucket runs beside the backward kernels
            // still to come [PTD-notes §2.2.3], which compete with it for the
            // CUs: it takes the shape for that. The last launch waits for the
            // backward's final kernels and then runs alone (the exposed tail):
            // it takes the shape tuned for bandwidth. Whether the queued work
            // is a backward or only the wait the last ddp_finish left there,
            // HIP cannot tell; a backward is the case that matters.
            r->beside_backward = b1 < r->pv.B;
            e = hipEventRecord(r->ev_ready, r->compute);
            if (e == hipSuccess) e = hipStreamWaitEvent(r->comm, r->ev_ready, 0);
        }
        if (e != hipSuccess) return hip_fail("stream wait", e);
    }
    int urc = upload_masks(r);
    if (urc != DDP_OK) return urc;
    if (r->hook) {
        for (int32_t b = b0; b < b1; ++b) {
            *at = b;
            int rc = r->hook(r->hook_ctx, b);
            if (rc != 0) return fail(DDP_ERR_HOOK, "communication hook returned " + std::to_string(rc) +
                                                       " for bucket " + std::to_string(b));
        }
        return DDP_OK;
    }
    if (!r->device) return fail(DDP_ERR_INVALID, "no device buffers and no communication hook");
    return enqueue_reduce(r, b0, b1, r->comm);
}

// Launch of buckets [b0, b1), which r->next has already moved past. A failed
// launch ends the backward's reductions: its error is returned here, every
// later launch of the backward is refused with the same code, and ddp_finish
// reports the buckets that were not reduced.
int launch_buckets(ddp_reducer *r, int32_t b0, int32_t b1)
{
    if (b0 >= b1) return DDP_OK;
    if (r->failed_bucket >= 0)
        return fail(r->failed_code, "buckets " + std::to_string(b0) + ".." + std::to_string(b1 - 1) +
                                        " not launched: the launch of bucket " + std::to_string(r->failed_bucket) +
                                        " failed earlier in this backward");
    int32_t at = b0;
    int rc;
    try {   // next already moved past these buckets: a throw must still count as a failed launch
        rc = issue_buckets(r, b0, b1, &at);
    } catch (const std::bad_alloc &) {
        rc = fail(DDP_ERR_NOMEM, kNoMemText);
    } catch (...) {
        rc = fail(DDP_ERR_INVALID, "internal error: unexpected exception while launching buckets");
    }
    if (rc != DDP_OK) {
        r->failed_bucket = at;
        r->failed_code = rc;
        try {
            r->failed_msg.assign(ddp_last_error());
        } catch (...) {
            r->failed_msg.clear();
        }
    }
    return rc;
}

// One gradient-ready mark [DDP-ch17 §17.12]: advances r->next past every
// bucket that is now launchable, in index order [L15 §2.3]; the caller
// launches [old next, new next).
void mark_state(ddp_reducer *r, int32_t param)
{
    r->ready[param] = 1;
    r->ready_order.push_back(param);
    ++r->marks;
    const int32_t b = r->pv.bucket_of[param];
    --r->pending[b];
    --r->group_pending[r->group_of[b]];
}

int mark_one(ddp_reducer *r, int32_t param)
{
    if (param < 0 || param >= r->pv.P) return fail(DDP_ERR_INVALID, "gradient index out of range");
    if (!r->sync) return DDP_OK;   // hooks are disabled inside no_sync [L15 §4.1; PTD-notes §2.2.4]
    if (r->marks == 0 && r->pv.find_unused) {
        // first hook of the backward: gradients no replica used are ready now
        // [DDP-ch17 §17.33]
        r->compute_masks();
        for (int32_t q = 0; q < r->pv.P; ++q)
            if (r->masks[q] == 0 && q != param) mark_state(r, q);
    }
    if (r->ready[param])
        return fail(DDP_ERR_ALREADY_READY, "Expected to mark a variable ready only once: gradient " +
                                               std::to_string(param) + " was marked ready twice in this backward pass");
    mark_state(r, param);
    r->advance();
    return DDP_OK;
}

void destroy_events(ddp_reducer *r) noexcept
{
    for (auto &ev : r->stage_ev)
        if (ev) {
            (void)hipEventSynchronize(ev);
            (void)hipEventDestroy(ev);
            ev = nullptr;
        }
    if (r->stage) (void)hipHostFree(r->stage);
    r->stage = nullptr;
    if (r->ev_ready) (void)hipEventDestroy(r->ev_ready);
    if (r->ev_done) (void)hipEventDestroy(r->ev_done);
    if (r->ev_host) (void)hipEventDestroy(r->ev_host);
    if (r->ev_tables) (void)hipEventDestroy(r->ev_tables);
    if (r->ev_foreign) (void)hipEventDestroy(r->ev_foreign);
    r->ev_tables = r->ev_foreign = nullptr;
    for (int i = 0; i < kTimingSlots; ++i) {
        if (r->ring0[i]) (void)hipEventDestroy(r->ring0[i]);
        if (r->ring1[i]) (void)hipEventDestroy(r->ring1[i]);
        r->ring0[i] = r->ring1[i] = nullptr;
    }
    r->ev_ready = r->ev_done = r->ev_host = nullptr;
}

// Deleter of a reducer: its events and staging, then the object.
struct ReducerRelease {
    void operator()(ddp_reducer *r) const noexcept
    {
        if (!r) return;
        destroy_events(r);
        delete r;
    }
};

}  // namespace

namespace {

// The entry points' bodies; the extern "C" definitions below run each one
// through guarded().


int ddp_plan_buckets_impl(int32_t n_params, const int64_t *param_bytes, const int32_t *order, int32_t order_mode,
                     int64_t cap_bytes, int64_t first_cap_bytes, int32_t *bucket_of, int64_t *offset_in_bucket,
                     int32_t *bucket_params, int32_t *bucket_nparams, int64_t *bucket_bytes, int32_t *n_buckets)
{
    if (!n_buckets) return fail(DDP_ERR_INVALID, "n_buckets is NULL");
    if (n_params < 0 || (n_params > 0 && !param_bytes)) return fail(DDP_ERR_INVALID, "bad gradient sizes");
    if (cap_bytes < 0 || first_cap_bytes < 0) return fail(DDP_ERR_INVALID, "caps must be non-negative");
    int64_t total = 0;   // every bucket's bytes are at most the total: checked once here
    for (int32_t p = 0; p < n_params; ++p) {
        if (param_bytes[p] < 0) return fail(DDP_ERR_INVALID, "gradient sizes must be non-negative");
        if (param_bytes[p] > std::numeric_limits<int64_t>::max() - total)
            return fail(DDP_ERR_INVALID, "gradient sizes add up to more than 2^63 bytes");
        total += param_bytes[p];
    }

    // the walk order [DDP-ch17 §17.3.1, §17.13; L15 §2.2]
    std::vector<int32_t> walk(n_params);
    if (order_mode == DDP_ORDER_REVERSE) {
        for (int32_t i = 0; i < n_params; ++i) walk[i] = n_params - 1 - i;
    } else if (order_mode == DDP_ORDER_FWD_THEN_REVERSE) {
        for (int32_t i = 0; i < n_params; ++i) walk[i] = i;
    } else if (order_mode == DDP_ORDER_GIVEN) {
        if (n_params > 0 && !order) return fail(DDP_ERR_INVALID, "order is NULL");
        std::vector<uint8_t> seen(n_params, 0);
        for (int32_t i = 0; i < n_params; ++i) {
            if (order[i] < 0 || order[i] >= n_params || seen[order[i]])
                return fail(DDP_ERR_INVALID, "order is not a permutation of the gradient indices");
            seen[order[i]] = 1;
            walk[i] = order[i];
        }
    } else {
        return fail(DDP_ERR_INVALID, "unknown order mode");
    }

    // seal a bucket once its bytes reach its cap [DDP-ch17 §17.2; L15 §8 exercise 3]
    std::vector<std::vector<int32_t>> buckets;
    std::vector<int32_t> open;
    int64_t open_bytes = 0;
    for (int32_t p : walk) {
        open.push_back(p);
        open_bytes += param_bytes[p];
        if (open_bytes >= (buckets.empty() ? first_cap_bytes : cap_bytes)) {
            buckets.push_back(std::move(open));
            open.clear();
            open_bytes = 0;
        }
    }
    if (!open.empty()) buckets.push_back(std::move(open));
    if (order_mode == DDP_ORDER_FWD_THEN_REVERSE) std::reverse(buckets.begin(), buckets.end());

    int32_t k = 0;
    for (size_t b = 0; b < buckets.size(); ++b) {
        int64_t off = 0;
        for (int32_t p : buckets[b]) {
            if (bucket_of) bucket_of[p] = int32_t(b);
            if (offset_in_bucket) offset_in_bucket[p] = off;
            if (bucket_params) bucket_params[k] = p;
            ++k;
            off += param_bytes[p];
        }
        if (bucket_nparams) bucket_nparams[b] = int32_t(buckets[b].size());
        if (bucket_bytes) bucket_bytes[b] = off;
    }
    *n_buckets = int32_t(buckets.size());
    return DDP_OK;
}

size_t ddp_workspace_bytes_impl(const ddp_reducer_desc *desc)
{
    PlanView pv;
    if (validate(desc, pv) != DDP_OK) return 0;
    if (build_segments(pv, pv.mode != DDP_IN_F32_VIEW || pv.find_unused) != DDP_OK) return 0;
    return layout_of(pv).total;
}

// Creation shared by ddp_reducer_create (tables in the caller's workspace)
// and ddp_reducer_create_static (tables in the library's static area).
int create_reducer(const ddp_reducer_desc *desc, ddp_reducer **out, bool static_area)
{
    if (!out) return fail(DDP_ERR_INVALID, "out is NULL");
    // released with its events and staging on every early return, and when
    // an allocation throws
    std::unique_ptr<ddp_reducer, ReducerRelease> r(new (std::nothrow) ddp_reducer());
    if (!r) return fail(DDP_ERR_NOMEM, kNoMemText);
    int rc = validate(desc, r->pv);
    if (rc != DDP_OK) return rc;
    if (r->pv.find_unused) {   // sized once: later updates of the tables allocate nothing
        r->window.assign(size_t(r->pv.W) * r->pv.P, 0);
        r->masks.assign(r->pv.P, 0);
    }
    PlanView &pv = r->pv;
    r->scale.s = 1.0f / float(pv.W);
    r->scale.w = float(pv.W);
    r->scale.divide = (pv.W & (pv.W - 1)) != 0;   // W not a power of two
    r->device = desc->flat != nullptr;
    r->compute = static_cast<hipStream_t>(desc->compute_stream);
    r->comm = static_cast<hipStream_t>(desc->comm_stream);
    if (r->device) {
        const bool copy_src = pv.mode != DDP_IN_F32_VIEW;
        rc = build_segments(pv, copy_src || pv.find_unused);
        if (rc != DDP_OK) return rc;
        for (int w = 0; w < pv.W; ++w)
            if (!desc->flat[w]) return fail(DDP_ERR_INVALID, "flat buffer of replica " + std::to_string(w) + " is NULL");
        if (copy_src) {
            if (pv.P > 0 && !desc->grads) return fail(DDP_ERR_INVALID, "gradient pointer table is NULL");
            for (int w = 0; w < pv.W; ++w)
                for (int32_t p = 0; p < pv.P; ++p)
                    if (pv.numel[p] > 0 && !desc->grads[size_t(w) * pv.P + p])
                        return fail(DDP_ERR_INVALID, "gradient pointer is NULL");
        }
        const Layout lay = layout_of(pv);
        void *workspace = desc->workspace;
        size_t workspace_bytes = desc->workspace_bytes;
        if (static_area) {
            // Unused detection stages its masks through pinned host memory,
            // which this variant does not allocate.
            if (pv.find_unused)
                return fail(DDP_ERR_INVALID, "ddp_reducer_create_static does not support unused-parameter "
                                             "detection (its mask staging would allocate pinned memory)");
            int dev = -1;
            hipError_t e = hipGetDevice(&dev);
            if (e == hipSuccess) e = ddp::static_table_area(dev, &workspace, &workspace_bytes);
            if (e != hipSuccess) return hip_fail("static table area", e);
            if (lay.total > workspace_bytes)
                return fail(DDP_ERR_INVALID, "the reducer's tables need " + std::to_string(lay.total) +
                                                 " bytes; the static table area holds " +
                                                 std::to_string(workspace_bytes) + " (DDP_STATIC_TABLE_BYTES)");
            r->static_device = dev;
        }
        if (!workspace || workspace_bytes < lay.total || reinterpret_cast<uintptr_t>(workspace) % 16)
            return fail(DDP_ERR_INVALID, "workspace missing, misaligned or smaller than " +
                                             std::to_string(lay.total) + " bytes");
        // Vector body of a segment: it starts at the first element whose
        // destination address is 256-byte aligned, so every wave's 1 KiB store
        // run covers whole cache lines (a store run that straddles lines costs
        // partial-line writes, up to a tenth of the bandwidth); the elements
        // before it are folded one per lane. This needs every replica's flat
        // buffer at the same address modulo 256; otherwise the body starts at
        // 16-byte alignment. Sources must then be 16-byte aligned at the body
        // start on every replica, else the segment is folded one element per
        // lane.
        const uintptr_t d0 = reinterpret_cast<uintptr_t>(desc->flat[0]);
        bool flat_aligned = d0 % 16 == 0, same_phase = true;
        for (int w = 0; w < pv.W; ++w) {
            flat_aligned &= reinterpret_cast<uintptr_t>(desc->flat[w]) % 16 == 0;
            same_phase &= reinterpret_cast<uintptr_t>(desc->flat[w]) % 256 == d0 % 256;
        }
        const uintptr_t line = same_phase ? 256 : 16;
        for (DeviceSeg &s : pv.segs) {
            if (!flat_aligned) continue;
            const uintptr_t a = d0 + 4 * uintptr_t(s.flat);
            int64_t head = int64_t(((line - a % line) % line) / 4);
            head = std::min(head, s.len);
            bool ok = true;
            if (copy_src) {
                const uintptr_t vec = pv.mode == DDP_IN_BF16_ACCUM_F32 ? 8 : 16;
                const uintptr_t esz = pv.mode == DDP_IN_BF16_ACCUM_F32 ? 2 : 4;
                for (int w = 0; w < pv.W && ok; ++w) {
                    uintptr_t a = reinterpret_cast<uintptr_t>(desc->grads[size_t(w) * pv.P + s.param]);
                    ok = (a + esz * uintptr_t(s.src + head)) % vec == 0;
                }
            }
            if (ok) s.head = int32_t(head);
        }
        std::vector<uint8_t> host(lay.total, 0);
        if (copy_src)
            std::memcpy(host.data() + lay.grads_off, desc->grads, sizeof(void *) * size_t(pv.W) * pv.P);
        std::memcpy(host.data() + lay.flat_off, desc->flat, sizeof(float *) * size_t(pv.W));
        std::memcpy(host.data() + lay.segs_off, pv.segs.data(), sizeof(DeviceSeg) * pv.segs.size());
        std::memcpy(host.data() + lay.tiles_off, pv.tile_seg.data(), sizeof(int32_t) * pv.tile_seg.size());
        if (pv.find_unused) {
            r->compute_masks();   // nothing recorded yet: every replica contributes
            r->segment_records(reinterpret_cast<DeviceSeg *>(host.data() + lay.segs_off));
            r->device_masks = r->masks;
        }
        // a static reducer claims the area before writing it: any earlier
        // static reducer on this device refuses to launch from here on
        hipError_t e = hipSuccess;
        if (static_area) {
            // reductions already queued by an earlier static reducer may still
            // read the area: let the device drain before it is rewritten
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return hip_fail("waiting for the device before rewriting the static table area", e);
            r->static_generation = ddp::claim_static_table_area(r->static_device);
        }
        e = hipMemcpy(workspace, host.data(), lay.total, hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail("workspace upload", e);
        uint8_t *ws = static_cast<uint8_t *>(workspace);
        r->tables.grads = copy_src ? reinterpret_cast<const void *const *>(ws + lay.grads_off) : nullptr;
        r->tables.flat = reinterpret_cast<float *const *>(ws + lay.flat_off);
        r->segs_dev = reinterpret_cast<DeviceSeg *>(ws + lay.segs_off);
        r->tables.segs = r->segs_dev;
        r->tables.tile_seg = reinterpret_cast<const int32_t *>(ws + lay.tiles_off);
        r->tables.n_params = pv.P;
        r->tables.masked = pv.find_unused ? 1 : 0;
        int dev = 0;
        e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&r->lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&r->lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&r->ev_ready, hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&r->ev_done, hipEventDisableTiming | hipEventDisableSystemFence);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&r->ev_host, hipEventDisableTiming);
        if (e == hipSuccess && pv.find_unused && !pv.segs.empty()) {
            e = hipHostMalloc(reinterpret_cast<void **>(&r->stage), 2 * sizeof(DeviceSeg) * pv.segs.size());
            for (int k = 0; k < 2 && e == hipSuccess; ++k)
                e = hipEventCreateWithFlags(&r->stage_ev[k], hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&r->ev_tables, hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&r->ev_foreign, hipEventDisableTiming);
        }
        if (e != hipSuccess) return hip_fail("reducer setup (device attributes, events, staging)", e);
    }
    r->ready_order.reserve(size_t(pv.P));   // a backward's marks then allocate nothing
    r->set_groups(nullptr, 0);
    r->reset();
    *out = r.release();
    return DDP_OK;
}

int ddp_reducer_create_impl(const ddp_reducer_desc *desc, ddp_reducer **out)
{
    return create_reducer(desc, out, false);
}

int ddp_reducer_create_static_impl(const ddp_reducer_desc *desc, ddp_reducer **out)
{
    return create_reducer(desc, out, true);
}

int ddp_reducer_destroy_impl(ddp_reducer *r)
{
    if (!r) return DDP_OK;
    // reductions still queued on the comm stream read and write the caller's
    // buffers: wait for them, so the buffers may be freed once this returns
    hipError_t e = hipSuccess;
    if (r->device && r->ev_host) {
        e = hipEventRecord(r->ev_host, r->comm);
        if (e == hipSuccess) e = hipEventSynchronize(r->ev_host);
    }
    ReducerRelease()(r);
    return e == hipSuccess ? DDP_OK : hip_fail("waiting for outstanding reductions", e);
}

int ddp_prepare_for_backward_impl(ddp_reducer *r)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (r->in_iteration())
        return fail(DDP_ERR_UNFINISHED,
                    "Expected to have finished reduction in the prior iteration before starting a new one. "
                    "Parameter indices which did not receive grad: " + list_params(r->unready()));
    if (r->failed_bucket >= 0 && !r->finished) r->end_window();   // a failed backward never finished
    r->reset();
    r->sync = r->require_sync;
    return DDP_OK;
}

int ddp_mark_ready_impl(ddp_reducer *r, int32_t param)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    const int32_t b0 = r->next;
    int rc = mark_one(r, param);
    if (rc != DDP_OK) return rc;
    return launch_buckets(r, b0, r->next);
}

int ddp_mark_ready_many_impl(ddp_reducer *r, const int32_t *params, int32_t n, int32_t *n_done)
{
    if (n_done) *n_done = 0;
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (n < 0 || (n > 0 && !params)) return fail(DDP_ERR_INVALID, "bad parameter list");
    const int32_t b0 = r->next;
    int rc = DDP_OK;
    for (int32_t i = 0; i < n && rc == DDP_OK; ++i) {
        rc = mark_one(r, params[i]);
        if (rc == DDP_OK && n_done) *n_done = i + 1;
    }
    // buckets completed by the marks that succeeded are launched even when a
    // later mark failed; the first error is the one reported
    const std::string err = rc != DDP_OK ? std::string(ddp_last_error()) : std::string();
    const int lrc = launch_buckets(r, b0, r->next);
    if (rc != DDP_OK) return fail(rc, err);
    return lrc;
}

int ddp_bucket_reduce_impl(ddp_reducer *r, int32_t bucket, void *stream)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (bucket < 0 || bucket >= r->pv.B) return fail(DDP_ERR_INVALID, "bucket index out of range");
    if (r->in_iteration() && bucket >= r->next)
        return fail(DDP_ERR_ORDER, "bucket " + std::to_string(bucket) + " still waits for gradients");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // With unused detection the segment table (it carries the replica masks)
    // is rewritten on the comm stream once per synchronized backward. A
    // reduction on another stream is ordered after the last rewrite, and the
    // next rewrite after it.
    const bool foreign = r->device && r->pv.find_unused && s != r->comm;
    hipError_t e = hipSuccess;
    if (r->device && r->pv.find_unused) {
        bool captured = false;
        if ((e = is_captured(s, &captured)) != hipSuccess) return hip_fail("stream capture status", e);
        if (captured)
            return fail(DDP_ERR_INVALID, "unused-parameter detection is not available while the stream is "
                                         "captured into a graph (the replica masks are host state)");
    }
    if (foreign) {
        e = hipEventRecord(r->ev_tables, r->comm);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, r->ev_tables, 0);
        if (e != hipSuccess) return hip_fail("ordering a reduction after the mask upload", e);
    }
    const int rc = enqueue_reduce(r, bucket, bucket + 1, s);
    if (rc != DDP_OK || !foreign) return rc;
    e = hipEventRecord(r->ev_foreign, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(r->comm, r->ev_foreign, 0);
    if (e != hipSuccess) return hip_fail("ordering the next mask upload after a reduction", e);
    return DDP_OK;
}

int ddp_finish_impl(ddp_reducer *r, int32_t host_blocking)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (host_blocking && r->device) {
        bool captured = false;
        const hipError_t e = is_captured(r->compute, &captured);
        if (e != hipSuccess) return hip_fail("stream capture status", e);
        if (captured)
            return fail(DDP_ERR_INVALID, "a host-blocking finish cannot wait while the compute stream is "
                                         "captured into a graph; nothing was changed");
    }
    if (!r->sync) {           // no_sync: nothing was reduced, the used tables keep accumulating
        r->finished = true;
        return DDP_OK;
    }
    if (r->failed_bucket >= 0) {
        r->finished = true;
        r->end_window();
        return fail(r->failed_code, "buckets " + std::to_string(r->failed_bucket) + ".." +
                                        std::to_string(r->pv.B - 1) + " of this backward were not reduced: " +
                                        r->failed_msg);
    }
    if (r->pv.find_unused && r->marks == 0 && r->next < r->pv.B) {
        // a backward in which no hook fired: every gradient unused everywhere
        // still completes, as at a first hook
        r->compute_masks();
        bool all_unused = true;
        for (uint64_t m : r->masks) all_unused &= m == 0;
        if (all_unused) {
            const int32_t b0 = r->next;
            for (int32_t q = 0; q < r->pv.P; ++q) mark_state(r, q);
            r->advance();
            int lrc = launch_buckets(r, b0, r->next);
            if (lrc != DDP_OK) return lrc;
        }
    }
    if (r->next < r->pv.B)
        return fail(DDP_ERR_NOT_READY, "Backward ended with buckets never reduced. "
                                       "Parameter indices which did not receive grad: " + list_params(r->unready()));
    if (r->device) {
        hipError_t e = hipSuccess;
        if (r->compute != r->comm) {
            e = hipEventRecord(r->ev_done, r->comm);
            if (e == hipSuccess) e = hipStreamWaitEvent(r->compute, r->ev_done, 0);
        }
        if (e == hipSuccess && host_blocking) {
            e = hipEventRecord(r->ev_host, r->comm);
            if (e == hipSuccess) e = hipEventSynchronize(r->ev_host);
        }
        if (e != hipSuccess) return hip_fail("finish", e);
    }
    r->finished = true;
    r->end_window();
    return DDP_OK;
}

int ddp_set_require_sync_impl(ddp_reducer *r, int32_t sync)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    r->require_sync = sync != 0;
    return DDP_OK;
}

int ddp_set_local_used_impl(ddp_reducer *r, const uint8_t *used)
{
    if (!r || !used) return fail(DDP_ERR_INVALID, "NULL argument");
    if (!r->pv.find_unused) return fail(DDP_ERR_INVALID, "unused-parameter detection is off for this reducer");
    if (r->sync && r->marks > 0)
        return fail(DDP_ERR_INVALID, "the used table must be set before the first gradient of the backward");
    // bounds in locals: a byte store may alias the vector's own pointers, so
    // a loop on window.size() would reload them after every element
    uint8_t *win = r->window.data();
    const size_t n = r->window.size();
    for (size_t i = 0; i < n; ++i) win[i] |= uint8_t(used[i] != 0);
    r->window_set = true;
    return DDP_OK;
}

int ddp_register_comm_hook_impl(ddp_reducer *r, ddp_comm_hook_fn fn, void *ctx)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    r->hook = fn;
    r->hook_ctx = ctx;
    return DDP_OK;
}

int ddp_set_bucket_groups_impl(ddp_reducer *r, const int32_t *first_bucket, int32_t n_groups)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (r->in_iteration())
        return fail(DDP_ERR_UNFINISHED, "cannot regroup buckets while a backward is in flight");
    if (n_groups < 0 || (n_groups > 0 && !first_bucket)) return fail(DDP_ERR_INVALID, "bad group list");
    if (n_groups > 0) {
        if (r->pv.B == 0 || first_bucket[0] != 0) return fail(DDP_ERR_INVALID, "the first group must start at bucket 0");
        for (int32_t g = 0; g < n_groups; ++g) {
            if (first_bucket[g] < 0 || first_bucket[g] >= r->pv.B || (g > 0 && first_bucket[g] <= first_bucket[g - 1]))
                return fail(DDP_ERR_INVALID, "group starts must be strictly increasing bucket indices");
        }
    }
    r->set_groups(n_groups > 0 ? first_bucket : nullptr, n_groups);
    r->count_groups();
    return DDP_OK;
}

int ddp_set_workgroups_per_cu_impl(ddp_reducer *r, int32_t n)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (n > 8) return fail(DDP_ERR_INVALID, "workgroups per CU must be at most 8 (or 0: automatic, < 0: no cap)");
    r->workgroups_per_cu = n;
    return DDP_OK;
}

int ddp_get_launch_lds_impl(const ddp_reducer *r, int32_t *lds_bytes)
{
    if (!r || !lds_bytes) return fail(DDP_ERR_INVALID, "NULL argument");
    *lds_bytes = int32_t(r->launch_lds());
    return DDP_OK;
}

int ddp_register_builtin_hook_impl(ddp_reducer *r, int32_t hook)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (hook != DDP_HOOK_ALLREDUCE && hook != DDP_HOOK_BF16_COMPRESS && hook != DDP_HOOK_FP16_COMPRESS)
        return fail(DDP_ERR_INVALID, "unknown built-in hook " + std::to_string(hook));
    if (r->in_iteration())
        return fail(DDP_ERR_UNFINISHED, "cannot change the hook while a backward is in flight");
    r->builtin_hook = hook;
    return DDP_OK;
}

int ddp_get_bucket_impl(const ddp_reducer *r, int32_t bucket, int64_t *bytes, int64_t *flat_offset_bytes,
                   int32_t *n_params)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (bucket < 0 || bucket >= r->pv.B) return fail(DDP_ERR_INVALID, "bucket index out of range");
    if (bytes) *bytes = r->pv.bucket_bytes[bucket];
    if (flat_offset_bytes) *flat_offset_bytes = r->pv.bucket_flat[bucket];
    if (n_params) *n_params = int32_t(r->pv.members[bucket].size());
    return DDP_OK;
}

int ddp_get_bucket_params_impl(const ddp_reducer *r, int32_t bucket, int32_t *params)
{
    if (!r || !params) return fail(DDP_ERR_INVALID, "NULL argument");
    if (bucket < 0 || bucket >= r->pv.B) return fail(DDP_ERR_INVALID, "bucket index out of range");
    std::copy(r->pv.members[bucket].begin(), r->pv.members[bucket].end(), params);
    return DDP_OK;
}

int ddp_get_ready_order_impl(const ddp_reducer *r, int32_t *order, int32_t *n)
{
    if (!r || !n) return fail(DDP_ERR_INVALID, "NULL argument");
    *n = int32_t(r->ready_order.size());
    if (order) std::copy(r->ready_order.begin(), r->ready_order.end(), order);
    return DDP_OK;
}

int ddp_get_launched_impl(const ddp_reducer *r, int32_t *n_launched)
{
    if (!r || !n_launched) return fail(DDP_ERR_INVALID, "NULL argument");
    *n_launched = r->next;
    return DDP_OK;
}

int ddp_set_timing_impl(ddp_reducer *r, int32_t enable)
{
    if (!r) return fail(DDP_ERR_INVALID, "reducer is NULL");
    if (!r->device) return fail(DDP_ERR_INVALID, "reducer has no device");
    r->timing = enable != 0;
    if (r->timing) {
        r->timed.clear();
        r->timed_resolved = 0;
    }
    return DDP_OK;
}

int ddp_get_timings_impl(const ddp_reducer *r, int32_t *first_bucket, int32_t *n_buckets, float *ms, int32_t capacity,
                    int32_t *n)
{
    if (!r || !n || capacity < 0) return fail(DDP_ERR_INVALID, "bad argument");
    if (r->timed.size() > size_t(std::numeric_limits<int32_t>::max()))
        return fail(DDP_ERR_INVALID, "more timing records than an int32 count holds");
    *n = int32_t(r->timed.size());
    const int32_t m = std::min(capacity, *n);
    if (ms && m > 0) {
        const int rc = resolve_timings(r, size_t(m));
        if (rc != DDP_OK) return rc;
    }
    for (int32_t i = 0; i < m; ++i) {
        if (first_bucket) first_bucket[i] = r->timed[i].first;
        if (n_buckets) n_buckets[i] = r->timed[i].count;
        if (ms) ms[i] = r->timed[i].ms;
    }
    return DDP_OK;
}

}  // namespace

extern "C" {

const char *ddp_last_error(void) { return g_err_fixed ? g_err_fixed : g_err.c_str(); }

int ddp_plan_buckets(int32_t n_params, const int64_t *param_bytes, const int32_t *order, int32_t order_mode, int64_t cap_bytes, int64_t first_cap_bytes, int32_t *bucket_of, int64_t *offset_in_bucket, int32_t *bucket_params, int32_t *bucket_nparams, int64_t *bucket_bytes, int32_t *n_buckets)
{
    return guarded([&] { return ddp_plan_buckets_impl(n_params, param_bytes, order, order_mode, cap_bytes, first_cap_bytes, bucket_of, offset_in_bucket, bucket_params, bucket_nparams, bucket_bytes, n_buckets); });
}

size_t ddp_workspace_bytes(const ddp_reducer_desc *desc)
{
    size_t n = 0;
    guarded([&] {
        n = ddp_workspace_bytes_impl(desc);
        return DDP_OK;
    });
    return n;
}

int ddp_reducer_create(const ddp_reducer_desc *desc, ddp_reducer **out)
{
    return guarded([&] { return ddp_reducer_create_impl(desc, out); });
}

int ddp_reducer_create_static(const ddp_reducer_desc *desc, ddp_reducer **out)
{
    return guarded([&] { return ddp_reducer_create_static_impl(desc, out); });
}

int ddp_reducer_destroy(ddp_reducer *r)
{
    return guarded([&] { return ddp_reducer_destroy_impl(r); });
}

int ddp_prepare_for_backward(ddp_reducer *r)
{
    return guarded([&] { return ddp_prepare_for_backward_impl(r); });
}

int ddp_mark_ready(ddp_reducer *r, int32_t param)
{
    return guarded([&] { return ddp_mark_ready_impl(r, param); });
}

int ddp_mark_ready_many(ddp_reducer *r, const int32_t *params, int32_t n, int32_t *n_done)
{
    return guarded([&] { return ddp_mark_ready_many_impl(r, params, n, n_done); });
}

int ddp_bucket_reduce(ddp_reducer *r, int32_t bucket, void *stream)
{
    return guarded([&] { return ddp_bucket_reduce_impl(r, bucket, stream); });
}

int ddp_finish(ddp_reducer *r, int32_t host_blocking)
{
    return guarded([&] { return ddp_finish_impl(r, host_blocking); });
}

int ddp_set_require_sync(ddp_reducer *r, int32_t sync)
{
    return guarded([&] { return ddp_set_require_sync_impl(r, sync); });
}

int ddp_set_local_used(ddp_reducer *r, const uint8_t *used)
{
    return guarded([&] { return ddp_set_local_used_impl(r, used); });
}

int ddp_register_comm_hook(ddp_reducer *r, ddp_comm_hook_fn fn, void *ctx)
{
    return guarded([&] { return ddp_register_comm_hook_impl(r, fn, ctx); });
}

int ddp_set_bucket_groups(ddp_reducer *r, const int32_t *first_bucket, int32_t n_groups)
{
    return guarded([&] { return ddp_set_bucket_groups_impl(r, first_bucket, n_groups); });
}

int ddp_set_workgroups_per_cu(ddp_reducer *r, int32_t n)
{
    return guarded([&] { return ddp_set_workgroups_per_cu_impl(r, n); });
}

int ddp_get_launch_lds(const ddp_reducer *r, int32_t *lds_bytes)
{
    return guarded([&] { return ddp_get_launch_lds_impl(r, lds_bytes); });
}

int ddp_register_builtin_hook(ddp_reducer *r, int32_t hook)
{
    return guarded([&] { return ddp_register_builtin_hook_impl(r, hook); });
}

int ddp_get_bucket(const ddp_reducer *r, int32_t bucket, int64_t *bytes, int64_t *flat_offset_bytes, int32_t *n_params)
{
    return guarded([&] { return ddp_get_bucket_impl(r, bucket, bytes, flat_offset_bytes, n_params); });
}

int ddp_get_bucket_params(const ddp_reducer *r, int32_t bucket, int32_t *params)
{
    return guarded([&] { return ddp_get_bucket_params_impl(r, bucket, params); });
}

int ddp_get_ready_order(const ddp_reducer *r, int32_t *order, int32_t *n)
{
    return guarded([&] { return ddp_get_ready_order_impl(r, order, n); });
}

int ddp_get_launched(const ddp_reducer *r, int32_t *n_launched)
{
    return guarded([&] { return ddp_get_launched_impl(r, n_launched); });
}

int ddp_set_timing(ddp_reducer *r, int32_t enable)
{
    return guarded([&] { return ddp_set_timing_impl(r, enable); });
}

int ddp_get_timings(const ddp_reducer *r, int32_t *first_bucket, int32_t *n_buckets, float *ms, int32_t capacity, int32_t *n)
{
    return guarded([&] { return ddp_get_timings_impl(r, first_bucket, n_buckets, ms, capacity, n); });
}

}  // extern "C"
