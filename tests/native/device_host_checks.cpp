// The device path's host logic of libddp (reducer.cpp) against a host-only
// stand-in for the HIP runtime (fake_hip.cpp), built under AddressSanitizer
// and UndefinedBehaviorSanitizer. Checks:
//  * timing: the event pool is a fixed ring however many launches are
//    timed, and every record's duration comes from its own launch's events
//    (an event pair is read before it is recorded again);
//  * unused-parameter detection with a reduction on another stream: that
//    stream waits for the mask upload on the comm stream, and the comm
//    stream (so the next upload) waits for the reduction;
//  * stream capture (a HIP graph recorded from the compute stream): the
//    compute stream is never queried, every launch waits on it by an event,
//    finish joins the comm stream back, and what a replay could not honour
//    (timing, unused detection, a host-blocking finish) is refused before
//    anything is enqueued;
//  * host memory exhaustion: with operator new failing after k allocations,
//    every entry point returns DDP_OK or DDP_ERR_NOMEM, nothing leaks, no
//    event is left behind, and a launch that could not be issued is
//    reported by ddp_finish like any failed launch.
// usage: device_host_checks       exit status 0 when every check holds.
#include "ddp.h"
#include "fake_hip.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <random>
#include <string>
#include <vector>

#include "failing_new.h"

namespace {

int g_bad = 0;

void expect(bool ok, const std::string &what)
{
    if (!ok && g_bad++ < 30) std::fprintf(stderr, "FAILED: %s\n", what.c_str());
}

hipStream_t stream_id(uintptr_t k)
{
    return reinterpret_cast<hipStream_t>(k);
}

const hipStream_t kCompute = stream_id(0x1000), kComm = stream_id(0x2000), kOther = stream_id(0x3000);

// A small model with device "buffers" (host memory the fake never touches
// beyond the workspace upload) and its plan.
struct Model {
    int W, P;
    std::vector<int64_t> numel, bytes, offset;
    std::vector<int32_t> bucket_of;
    int32_t B = 0;
    std::vector<std::vector<float>> store;   // backing for gradient and flat pointers
    std::vector<const void *> grads;
    std::vector<float *> flat;
    std::vector<uint8_t> workspace;
    ddp_reducer_desc d{};

    Model(int W_, int P_, int64_t cap, bool find_unused, uint32_t seed) : W(W_), P(P_)
    {
        std::mt19937 rng(seed);
        numel.resize(P);
        bytes.resize(P);
        for (int p = 0; p < P; ++p) {
            numel[p] = 1 + int64_t(rng() % 3000);
            bytes[p] = 4 * numel[p];
        }
        bucket_of.resize(P);
        offset.resize(P);
        std::vector<int32_t> bparams(P), bn(P);
        std::vector<int64_t> bb(P);
        const int rc = ddp_plan_buckets(P, bytes.data(), nullptr, DDP_ORDER_REVERSE, cap, cap, bucket_of.data(),
                                        offset.data(), bparams.data(), bn.data(), bb.data(), &B);
        expect(rc == DDP_OK, "plan");
        int64_t total = 0;
        for (int b = 0; b < B; ++b) total += bb[b] / 4;
        for (int w = 0; w < W; ++w) {
            store.emplace_back(size_t(total) + 64);
            flat.push_back(store.back().data());
        }
        for (int w = 0; w < W; ++w)
            for (int p = 0; p < P; ++p) {
                store.emplace_back(size_t(numel[p]) + 4);
                grads.push_back(store.back().data());
            }
        d.world = W;
        d.n_params = P;
        d.param_numel = numel.data();
        d.bucket_of = bucket_of.data();
        d.offset_in_bucket = offset.data();
        d.n_buckets = B;
        d.input_mode = DDP_IN_F32_COPY;
        d.grads = grads.data();
        d.flat = flat.data();
        d.compute_stream = kCompute;
        d.comm_stream = kComm;
        d.collective = DDP_ALL_REDUCE;
        d.find_unused = find_unused ? 1 : 0;
        const size_t ws = ddp_workspace_bytes(&d);
        expect(ws > 0, "workspace bytes");
        workspace.assign(ws + 256, 0);
        uintptr_t a = reinterpret_cast<uintptr_t>(workspace.data());
        d.workspace = reinterpret_cast<void *>((a + 255) / 256 * 256);
        d.workspace_bytes = ws;
    }
};

// Every gradient ready, bucket by bucket (one launch per bucket).
int backward(ddp_reducer *r, const Model &m)
{
    int rc = ddp_prepare_for_backward(r);
    if (rc != DDP_OK) return rc;
    for (int p = m.P - 1; p >= 0; --p) {
        rc = ddp_mark_ready(r, p);
        if (rc != DDP_OK) return rc;
    }
    return ddp_finish(r, 0);
}

void check_timing_ring()
{
    fake::g_logging = false;
    const long live0 = fake::g_live_events;
    fake::g_max_live_events = live0;
    Model m(4, 40, 20000, false, 7);
    ddp_reducer *r = nullptr;
    expect(ddp_reducer_create(&m.d, &r) == DDP_OK, "timing: create");
    const long base = fake::g_live_events - live0;   // the reducer's stream-ordering events
    expect(ddp_set_timing(r, 1) == DDP_OK, "timing: enable");
    const int steps = 600;
    for (int s = 0; s < steps; ++s) expect(backward(r, m) == DDP_OK, "timing: backward");
    const long launches = long(steps) * m.B;
    expect(launches > 4 * 256, "timing: enough launches to wrap the ring several times");
    expect(fake::g_max_live_events - live0 <= base + 2 * 256,
           "timing: at most 256 event pairs alive (" + std::to_string(fake::g_max_live_events - live0) + ")");
    int32_t n = 0;
    expect(ddp_get_timings(r, nullptr, nullptr, nullptr, 0, &n) == DDP_OK && n == launches, "timing: record count");
    const size_t nn = size_t(n);
    std::vector<int32_t> first(nn), count(nn);
    std::vector<float> ms(nn);
    expect(ddp_get_timings(r, first.data(), count.data(), ms.data(), n, &n) == DDP_OK, "timing: read");
    // each record's duration is the stamp of its own start event: strictly
    // increasing when no pair was recorded again before it was read
    bool increasing = true, order = true;
    for (int32_t i = 0; i < n; ++i) {
        if (i > 0 && !(ms[i] > ms[i - 1])) increasing = false;
        if (first[i] != i % m.B || count[i] != 1) order = false;
    }
    expect(increasing, "timing: a record read another launch's events");
    expect(order, "timing: records out of launch order");
    // re-enabling starts a new list on the same ring
    expect(ddp_set_timing(r, 1) == DDP_OK && backward(r, m) == DDP_OK, "timing: second list");
    expect(ddp_get_timings(r, nullptr, nullptr, nullptr, 0, &n) == DDP_OK && n == m.B, "timing: second list count");
    expect(ddp_reducer_destroy(r) == DDP_OK, "timing: destroy");
    expect(fake::g_live_events == live0, "timing: events left after destroy");
    fake::g_logging = true;
}

struct HookCtx {
    ddp_reducer *r;
    hipStream_t s;
};

int reduce_on_other_stream(void *ctx, int32_t bucket)
{
    HookCtx *h = static_cast<HookCtx *>(ctx);
    return ddp_bucket_reduce(h->r, bucket, h->s) == DDP_OK ? 0 : 1;
}

void check_foreign_stream_masks()
{
    fake::reset_log();
    Model m(4, 12, 8000, true, 11);
    ddp_reducer *r = nullptr;
    expect(ddp_reducer_create(&m.d, &r) == DDP_OK, "masks: create");
    HookCtx h{r, kOther};
    expect(ddp_register_comm_hook(r, reduce_on_other_stream, &h) == DDP_OK, "masks: hook");
    std::vector<uint8_t> used(size_t(m.W) * m.P, 1);
    for (int it = 0; it < 3; ++it) {
        fake::reset_log();
        used[size_t(it % m.W) * m.P + size_t(it)] = 0;   // the masks change every iteration
        expect(ddp_prepare_for_backward(r) == DDP_OK, "masks: prepare");
        expect(ddp_set_local_used(r, used.data()) == DDP_OK, "masks: used");
        for (int p = m.P - 1; p >= 0; --p) expect(ddp_mark_ready(r, p) == DDP_OK, "masks: mark");
        expect(ddp_finish(r, 0) == DDP_OK, "masks: finish");
        // the upload (a copy on comm) comes first; every launch on the other
        // stream is preceded by that stream waiting on an event last recorded
        // on comm after the upload, and followed by comm waiting on an event
        // recorded on the other stream after the launch
        const auto &L = fake::g_log;
        size_t copy_at = L.size();
        for (size_t i = 0; i < L.size(); ++i)
            if (!std::strcmp(L[i].what, "copy")) {
                expect(L[i].stream == kComm, "masks: upload not on comm");
                if (copy_at == L.size()) copy_at = i;
            }
        expect(copy_at < L.size(), "masks: no upload although the masks changed");
        int launches = 0;
        for (size_t i = 0; i < L.size(); ++i) {
            if (std::strcmp(L[i].what, "launch")) continue;
            ++launches;
            expect(L[i].stream == kOther, "masks: launch not on the hook's stream");
            expect(i > copy_at, "masks: launch before the upload");
            bool waited = false;
            for (size_t j = i; j-- > copy_at;) {
                if (!std::strcmp(L[j].what, "wait") && L[j].stream == kOther) {
                    // its event was last recorded on comm, after the upload
                    for (size_t k = j; k-- > copy_at;)
                        if (!std::strcmp(L[k].what, "record") && L[k].event == L[j].event) {
                            waited = L[k].stream == kComm;
                            break;
                        }
                    break;
                }
            }
            expect(waited, "masks: the other stream did not wait for the upload");
            bool back = false;
            for (size_t j = i + 1; j + 1 < L.size() + 1 && j < L.size(); ++j) {
                if (!std::strcmp(L[j].what, "record") && L[j].stream == kOther) {
                    for (size_t k = j + 1; k < L.size(); ++k)
                        if (!std::strcmp(L[k].what, "wait") && L[k].event == L[j].event) {
                            back = L[k].stream == kComm;
                            break;
                        }
                    break;
                }
            }
            expect(back, "masks: comm did not wait for the reduction on the other stream");
        }
        expect(launches == m.B, "masks: one launch per bucket");
    }
    expect(ddp_reducer_destroy(r) == DDP_OK, "masks: destroy");
}

// Runs f with operator new failing after k allocations, for k = 0, 1, ...
// until f succeeds; each failing run must return DDP_ERR_NOMEM.
template <class F>
int until_success(const char *what, F f)
{
    for (long k = 0; k < 100000; ++k) {
        g_new_budget = k;
        const int rc = f();
        g_new_budget = -1;
        if (rc == DDP_OK) return int(k);
        if (rc != DDP_ERR_NOMEM) {
            expect(false, std::string(what) + ": status " + std::to_string(rc) + " under a failing allocation (" +
                              ddp_last_error() + ")");
            return -1;
        }
        expect(std::strlen(ddp_last_error()) > 0, std::string(what) + ": no error text");
    }
    expect(false, std::string(what) + ": never succeeded");
    return -1;
}

void check_out_of_memory()
{
    fake::g_logging = false;
    const long live0 = fake::g_live_events;
    for (int fu = 0; fu < 2; ++fu) {
        Model m(4, 30, 12000, fu == 1, 23);
        // plan
        std::vector<int32_t> bo(size_t(m.P)), bp(size_t(m.P)), bn(size_t(m.P));
        std::vector<int64_t> off(size_t(m.P)), bb(size_t(m.P));
        int32_t B = 0;
        int n_allocs = until_success("plan", [&] {
            return ddp_plan_buckets(m.P, m.bytes.data(), nullptr, DDP_ORDER_FWD_THEN_REVERSE, 12000, 4000,
                                    bo.data(), off.data(), bp.data(), bn.data(), bb.data(), &B);
        });
        expect(n_allocs >= 0, "plan under failing allocations");
        // workspace size
        for (long k = 0; k < 100000; ++k) {
            g_new_budget = k;
            const size_t ws = ddp_workspace_bytes(&m.d);
            g_new_budget = -1;
            if (ws) break;
            expect(std::strcmp(ddp_last_error(), "out of host memory") == 0, "workspace bytes: error text");
        }
        // create: every failure leaves nothing behind (events, staging, host state: ASan checks leaks)
        ddp_reducer *r = nullptr;
        bool clean = true;
        int created = until_success("create", [&] {
            r = nullptr;
            const int rc = ddp_reducer_create(&m.d, &r);
            if (rc != DDP_OK) clean &= r == nullptr && fake::g_live_events == live0;
            return rc;
        });
        expect(clean, "create: a failed create left state behind");
        expect(created > 0 && r != nullptr, "create under failing allocations");
        if (!r) continue;
        // a backward whose calls fail one allocation at a time: the failing
        // call returns NOMEM; a launch that could not be issued fails the
        // backward, which ddp_finish then reports; the next backward works
        expect(ddp_set_timing(r, 1) == DDP_OK, "oom: timing on");   // timing records allocate per launch
        bool finish_reported = false;
        for (long k = 0; k < 64; ++k) {
            expect(ddp_prepare_for_backward(r) == DDP_OK, "oom: prepare");
            if (fu) {
                std::vector<uint8_t> used(size_t(m.W) * m.P, 1);
                used[3] = 0;
                expect(ddp_set_local_used(r, used.data()) == DDP_OK, "oom: used");
            }
            std::vector<int> status(size_t(m.P), DDP_OK);   // checked once allocations succeed again
            g_new_budget = k;
            for (int p = m.P - 1; p >= 0; --p) status[size_t(p)] = ddp_mark_ready(r, p);
            const int frc = ddp_finish(r, 0);
            g_new_budget = -1;
            int failed = DDP_OK;
            for (int p = m.P - 1; p >= 0; --p) {
                const int rc = status[size_t(p)];
                if (rc != DDP_OK && failed == DDP_OK) failed = rc;
                expect(rc == DDP_OK || rc == DDP_ERR_NOMEM, "oom: mark status " + std::to_string(rc));
            }
            expect(frc == DDP_OK || frc == DDP_ERR_NOMEM, "oom: finish status " + std::to_string(frc));
            if (failed != DDP_OK) {
                expect(frc != DDP_OK, "oom: finish hid a launch that failed");
                finish_reported = true;
            }
            int32_t launched = -1;
            ddp_get_launched(r, &launched);
            if (frc == DDP_OK) expect(launched == m.B, "oom: finish succeeded with buckets unlaunched");
        }
        expect(finish_reported, "oom: no launch ever failed (the budget never reached a launch)");
        expect(backward(r, m) == DDP_OK, "oom: a later backward");
        // regrouping under failing allocations keeps the old groups intact
        std::vector<int32_t> firsts;
        for (int b = 0; b < m.B; b += 2) firsts.push_back(b);
        until_success("groups", [&] { return ddp_set_bucket_groups(r, firsts.data(), int32_t(firsts.size())); });
        expect(backward(r, m) == DDP_OK, "oom: backward after regrouping");
        expect(ddp_reducer_destroy(r) == DDP_OK, "oom: destroy");
        expect(fake::g_live_events == live0, "oom: events left after destroy");
    }
    fake::g_logging = true;
}

// ddp_reducer_create_static: the tables go to the static area (the
// workspace is ignored), the device drains before the area is rewritten, a
// later static reducer makes the earlier one refuse to launch, and unused
// detection and oversized tables are refused.
void check_static_area()
{
    fake::g_logging = true;
    Model a(4, 20, 8000, false, 31), b(2, 5, 1000, false, 32);
    a.d.workspace = nullptr;   // ignored by the static variant
    a.d.workspace_bytes = 0;
    b.d.workspace = nullptr;
    b.d.workspace_bytes = 0;
    ddp_reducer *ra = nullptr, *rb = nullptr;
    fake::reset_log();
    expect(ddp_reducer_create_static(&a.d, &ra) == DDP_OK && ra, "static: create");
    bool drained = false;
    for (const auto &c : fake::g_log) drained |= !std::strcmp(c.what, "device_sync");
    expect(drained, "static: the device was not drained before the area was written");
    expect(backward(ra, a) == DDP_OK, "static: backward");
    expect(ddp_reducer_create_static(&b.d, &rb) == DDP_OK && rb, "static: second create");
    expect(backward(rb, b) == DDP_OK, "static: second reducer's backward");
    int rc = backward(ra, a);
    expect(rc == DDP_ERR_INVALID && std::strstr(ddp_last_error(), "replaced"),
           "static: the first reducer launched from a replaced table area");
    expect(ddp_bucket_reduce(ra, 0, kComm) == DDP_ERR_INVALID, "static: explicit reduce from a replaced area");
    // a regular reducer is unaffected by the static area
    ddp_reducer *rr = nullptr;
    Model c(3, 7, 4000, false, 33);
    expect(ddp_reducer_create(&c.d, &rr) == DDP_OK && backward(rr, c) == DDP_OK, "static: regular reducer");
    // unused detection is refused
    Model u(2, 5, 1000, true, 34);
    ddp_reducer *ru = nullptr;
    expect(ddp_reducer_create_static(&u.d, &ru) == DDP_ERR_INVALID && !ru, "static: unused detection accepted");
    expect(ddp_reducer_destroy(ra) == DDP_OK && ddp_reducer_destroy(rb) == DDP_OK && ddp_reducer_destroy(rr) == DDP_OK,
           "static: destroy");
}

// The occupancy rule of a launch: the tuned cap (two workgroups per CU at
// W = 8) for back-to-back reductions and for the launch that holds the
// backward's last bucket (the exposed tail); one per CU, with two tiles per
// workgroup, for the other launches of a backward while the compute stream
// has work queued.
void check_launch_occupancy()
{
    fake::g_logging = true;
    Model m(8, 12, 6000, false, 41);   // several buckets: one launch per bucket
    expect(m.B >= 3, "occupancy: the model has several buckets");
    ddp_reducer *r = nullptr;
    expect(ddp_reducer_create(&m.d, &r) == DDP_OK, "occupancy: create");
    int32_t tuned = 0;
    expect(ddp_get_launch_lds(r, &tuned) == DDP_OK && tuned == 56832, "occupancy: two per CU at W = 8");
    const unsigned one = 83968;   // one per CU
    auto launches = [&](ddp_reducer *rr, const Model &mm) {
        fake::reset_log();
        std::vector<fake::Call> v;
        if (backward(rr, mm) != DDP_OK) return v;
        for (const auto &c : fake::g_log)
            if (!std::strcmp(c.what, "launch")) v.push_back(c);
        return v;
    };
    auto shape = [&](const std::vector<fake::Call> &v, unsigned lds_first, bool pair_first, unsigned lds_last,
                     bool pair_last) {
        if (v.size() != size_t(m.B)) return false;
        for (size_t i = 0; i + 1 < v.size(); ++i)
            if (v[i].lds != lds_first || v[i].pair != pair_first) return false;
        return v.back().lds == lds_last && v.back().pair == pair_last;
    };
    fake::g_stream_query = hipErrorNotReady;   // the compute stream has work queued
    expect(shape(launches(r, m), one, true, unsigned(tuned), false),
           "occupancy: beside a backward one per CU with two tiles, the last launch tuned");
    fake::g_stream_query = hipSuccess;         // compute drained: nothing runs beside
    expect(shape(launches(r, m), unsigned(tuned), false, unsigned(tuned), false),
           "occupancy: drained compute stream keeps the tuned cap");
    fake::g_stream_query = hipErrorNotReady;
    expect(ddp_set_workgroups_per_cu(r, 2) == DDP_OK &&
               shape(launches(r, m), unsigned(tuned), false, unsigned(tuned), false),
           "occupancy: explicit cap of two kept beside a backward");
    expect(ddp_set_workgroups_per_cu(r, 1) == DDP_OK && shape(launches(r, m), one, true, one, true),
           "occupancy: explicit cap of one: two tiles per workgroup");
    expect(ddp_set_workgroups_per_cu(r, -1) == DDP_OK && shape(launches(r, m), 0, false, 0, false),
           "occupancy: no cap");
    expect(ddp_reducer_destroy(r) == DDP_OK, "occupancy: destroy");
    // W = 16 (one vector group per thread, two per CU tuned) has no two-tile form
    Model m16(16, 12, 6000, false, 42);
    expect(ddp_reducer_create(&m16.d, &r) == DDP_OK, "occupancy: create W = 16");
    fake::g_stream_query = hipErrorNotReady;
    const auto v16 = launches(r, m16);
    bool ok = v16.size() == size_t(m16.B) && !v16.empty();
    for (size_t i = 0; ok && i < v16.size(); ++i) ok = !v16[i].pair && (i + 1 == v16.size()) == (v16[i].lds != one);
    expect(ok, "occupancy: W = 16 beside a backward: one per CU, single tiles");
    expect(ddp_reducer_destroy(r) == DDP_OK, "occupancy: destroy W = 16");
    fake::g_stream_query = hipErrorNotReady;
}

// Stream capture: the launch path must not query the compute stream (a
// query of a capturing stream breaks the capture). Each launch waits on the
// compute stream by an event, the launches of a backward but the last take
// the shape for running beside one, and finish makes the compute stream wait
// for the comm stream (the graph's join). Timing, unused detection and a
// host-blocking finish are refused with nothing enqueued.
void check_capture()
{
    fake::g_logging = true;
    Model m(8, 12, 6000, false, 41);
    ddp_reducer *r = nullptr;
    expect(ddp_reducer_create(&m.d, &r) == DDP_OK, "capture: create");
    int32_t tuned = 0;
    expect(ddp_get_launch_lds(r, &tuned) == DDP_OK, "capture: launch LDS");
    const unsigned one = 83968;   // one per CU
    fake::g_stream_query = hipSuccess;   // a query would (wrongly) report a drained stream
    fake::g_capturing = true;
    fake::g_stream_queries = 0;
    fake::reset_log();
    expect(backward(r, m) == DDP_OK, "capture: backward");
    expect(fake::g_stream_queries == 0, "capture: the compute stream was queried");
    int launches = 0, waits = 0;
    bool waited_before_each = true, shapes = true;
    bool compute_waited = false;
    for (size_t i = 0; i < fake::g_log.size(); ++i) {
        const fake::Call &c = fake::g_log[i];
        if (!std::strcmp(c.what, "wait") && c.stream == kComm) ++waits;
        if (!std::strcmp(c.what, "launch")) {
            waited_before_each &= waits == launches + 1 && c.stream == kComm;
            const bool last = launches == m.B - 1;
            shapes &= c.lds == (last ? unsigned(tuned) : one) && c.pair == !last;
            ++launches;
        }
        if (!std::strcmp(c.what, "wait") && c.stream == kCompute) compute_waited = launches == m.B;
    }
    expect(launches == m.B, "capture: one launch per bucket");
    expect(waited_before_each, "capture: every launch waits on the compute stream");
    expect(shapes, "capture: beside-backward shape but for the last launch");
    expect(compute_waited, "capture: finish joins the comm stream into the compute stream");

    // a host-blocking finish is refused and changes nothing
    expect(ddp_prepare_for_backward(r) == DDP_OK, "capture: prepare");
    for (int p = m.P - 1; p >= 0; --p) expect(ddp_mark_ready(r, p) == DDP_OK, "capture: mark");
    fake::reset_log();
    expect(ddp_finish(r, 1) == DDP_ERR_INVALID, "capture: host-blocking finish refused");
    expect(fake::g_log.empty(), "capture: the refused finish enqueued something");
    expect(ddp_finish(r, 0) == DDP_OK, "capture: finish without blocking after the refusal");

    // timing is refused at the first launch, before the wait
    expect(ddp_set_timing(r, 1) == DDP_OK, "capture: timing on");
    expect(ddp_prepare_for_backward(r) == DDP_OK, "capture: prepare (timing)");
    fake::reset_log();
    int rc = DDP_OK;
    for (int p = m.P - 1; p >= 0 && rc == DDP_OK; --p) rc = ddp_mark_ready(r, p);
    expect(rc == DDP_ERR_INVALID, "capture: timed launch refused");
    expect(fake::g_log.empty(), "capture: the refused launch enqueued something");
    expect(ddp_set_timing(r, 0) == DDP_OK, "capture: timing off");
    expect(ddp_prepare_for_backward(r) == DDP_OK, "capture: prepare after the refusal");
    expect(backward(r, m) == DDP_OK, "capture: backward after the refusal");
    expect(ddp_reducer_destroy(r) == DDP_OK, "capture: destroy");

    // unused-parameter detection is refused the same way
    Model mu(4, 10, 4000, true, 43);
    fake::g_capturing = false;
    expect(ddp_reducer_create(&mu.d, &r) == DDP_OK, "capture: create (unused detection)");
    fake::g_capturing = true;
    expect(ddp_prepare_for_backward(r) == DDP_OK, "capture: prepare (unused detection)");
    fake::reset_log();
    rc = DDP_OK;
    for (int p = mu.P - 1; p >= 0 && rc == DDP_OK; --p) rc = ddp_mark_ready(r, p);
    expect(rc == DDP_ERR_INVALID, "capture: unused detection refused");
    expect(fake::g_log.empty(), "capture: the refused launch (unused detection) enqueued something");
    expect(ddp_bucket_reduce(r, 0, kOther) == DDP_ERR_INVALID && fake::g_log.empty(),
           "capture: a standalone reduction with unused detection refused, nothing enqueued");
    fake::g_capturing = false;
    expect(ddp_reducer_destroy(r) == DDP_OK, "capture: destroy (unused detection)");
    fake::g_stream_query = hipErrorNotReady;
}

}  // namespace

int main()
{
    check_launch_occupancy();
    check_capture();
    check_timing_ring();
    check_foreign_stream_masks();
    check_out_of_memory();
    check_static_area();
    if (g_bad) {
        std::fprintf(stderr, "%d violations\n", g_bad);
        return 1;
    }
    std::printf("device_host_checks ok\n");
    return 0;
}
