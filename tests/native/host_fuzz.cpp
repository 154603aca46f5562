// Random API sequences against host-only reducers (no device buffers: every
// launch goes to a registered callback), for a build of reducer.cpp under
// AddressSanitizer and UndefinedBehaviorSanitizer. Besides the sanitizers'
// own checks it asserts the reducer's contract after every call:
//  * buckets reach the callback strictly in index order, each at most once
//    per backward, starting from bucket 0 after every prepare;
//  * ddp_get_launched agrees with the callbacks seen;
//  * after a failing callback nothing more launches in that backward, and
//    ddp_finish reports the failure;
//  * a successful ddp_finish of a synchronized backward saw every bucket;
//  * every status is one of the documented codes.
// With "oom", one call in ten runs with operator new failing after a few
// allocations: such a call may also return DDP_ERR_NOMEM, and every
// invariant above must still hold (a launch that could not be issued counts
// as a failed one).
// usage: host_fuzz SEEDS [oom]     exit status 0 when every sequence holds.
#include "ddp.h"

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <new>
#include <random>
#include <string>
#include <vector>

#include "failing_new.h"

namespace {

bool g_oom = false;

struct Recorder {
    std::vector<int32_t> seen;   // buckets handed to the callback in this backward
    int32_t fail_at = -1;        // bucket whose callback returns an error
    bool failed = false;
};

int on_bucket(void *ctx, int32_t bucket)
{
    Recorder *rec = static_cast<Recorder *>(ctx);
    rec->seen.push_back(bucket);
    if (bucket == rec->fail_at) {
        rec->failed = true;
        return 7;
    }
    return 0;
}

int g_bad = 0;

void expect(bool ok, const char *what, int seed, int step)
{
    if (!ok && g_bad++ < 20) std::fprintf(stderr, "seed %d step %d: %s\n", seed, step, what);
}

bool known_status(int rc)
{
    return rc == DDP_OK || rc == DDP_ERR_INVALID || rc == DDP_ERR_ALREADY_READY || rc == DDP_ERR_UNFINISHED ||
           rc == DDP_ERR_NOT_READY || rc == DDP_ERR_ORDER || rc == DDP_ERR_HIP || rc == DDP_ERR_HOOK ||
           (g_oom && rc == DDP_ERR_NOMEM);
}

void run(int seed)
{
    std::mt19937 rng(uint32_t(seed) * 2654435761u + 1);
    auto pick = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    const int P = pick(1, 30);
    const int W = pick(1, 8);
    std::vector<int64_t> numel(P), bytes(P);
    for (int p = 0; p < P; ++p) {
        numel[p] = pick(0, 40);
        bytes[p] = 4 * numel[p];
    }
    const int64_t caps[] = {0, 16, 64, 400, int64_t(1) << 40};
    const int64_t cap = caps[pick(0, 4)], first = caps[pick(0, 3)];
    const int mode = pick(0, 2);
    std::vector<int32_t> order(P);
    for (int p = 0; p < P; ++p) order[p] = p;
    std::shuffle(order.begin(), order.end(), rng);
    std::vector<int32_t> bucket_of(P), bparams(P), bn(P);
    std::vector<int64_t> offset(P), bbytes(P);
    int32_t B = 0;
    int rc = ddp_plan_buckets(P, bytes.data(), order.data(), mode, cap, first, bucket_of.data(), offset.data(),
                              bparams.data(), bn.data(), bbytes.data(), &B);
    expect(rc == DDP_OK && B >= 1 && B <= P, "plan", seed, -1);
    if (rc != DDP_OK) return;

    ddp_reducer_desc d{};
    d.world = W;
    d.n_params = P;
    d.param_numel = numel.data();
    d.bucket_of = bucket_of.data();
    d.offset_in_bucket = offset.data();
    d.n_buckets = B;
    d.input_mode = DDP_IN_F32_COPY;
    d.collective = pick(0, 1);
    d.find_unused = pick(0, 1);
    ddp_reducer *r = nullptr;
    rc = ddp_reducer_create(&d, &r);
    expect(rc == DDP_OK && r, "create", seed, -1);
    if (rc != DDP_OK) return;
    Recorder rec;
    rec.seen.reserve(size_t(B));   // the callback allocates nothing while allocations may fail
    ddp_register_comm_hook(r, on_bucket, &rec);

    bool sync = true, sync_next = true, prepared = false;
    std::vector<uint8_t> used(size_t(W) * P, 1);
    for (int step = 0; step < 200; ++step) {
        const int op = pick(0, 99);
        // the budget applies to the library call of this step only; the
        // checks after it allocate freely
        const long budget = g_oom && pick(0, 9) == 0 ? pick(0, 4) : -1;
        if (op < 10) {                                    // prepare
            g_new_budget = budget;
            rc = ddp_prepare_for_backward(r);
            g_new_budget = -1;
            expect(known_status(rc), "prepare status", seed, step);
            if (rc == DDP_OK) {
                rec.seen.clear();
                rec.failed = false;
                rec.fail_at = pick(0, 9) == 0 ? pick(0, B - 1) : -1;
                sync = sync_next;
                prepared = true;
            }
        } else if (op < 60) {                             // one mark, sometimes out of range or repeated
            const int p = pick(-1, P);
            g_new_budget = budget;
            rc = ddp_mark_ready(r, p);
            g_new_budget = -1;
            expect(known_status(rc), "mark status", seed, step);
        } else if (op < 75) {                             // a batch of marks
            std::vector<int32_t> batch(pick(0, 6));
            for (auto &x : batch) x = pick(0, P - 1);
            int32_t done = -1;
            g_new_budget = budget;
            rc = ddp_mark_ready_many(r, batch.data(), int32_t(batch.size()), &done);
            g_new_budget = -1;
            expect(known_status(rc) && done >= 0 && done <= int32_t(batch.size()), "mark_many status", seed, step);
        } else if (op < 85) {                             // finish
            const size_t before = rec.seen.size();
            g_new_budget = budget;
            rc = ddp_finish(r, 0);
            g_new_budget = -1;
            expect(known_status(rc), "finish status", seed, step);
            if (rc == DDP_OK && prepared && sync) {
                int32_t launched = -1;
                ddp_get_launched(r, &launched);
                expect(launched == B, "finish succeeded with buckets unlaunched", seed, step);
                // every bucket reached the callback: none was lost to a launch
                // that failed (a hook error, or an allocation failure)
                expect(rec.seen.size() == size_t(B), "finish succeeded with a bucket never handed to the hook",
                       seed, step);
            }
            if (rec.failed) expect(rc != DDP_OK || !sync, "finish hid a failed launch", seed, step);
            (void)before;
        } else if (op < 89) {                             // no_sync toggle, read at the next prepare
            sync_next = pick(0, 1) == 1;
            ddp_set_require_sync(r, sync_next ? 1 : 0);
        } else if (op < 93) {                             // used tables
            for (auto &u : used) u = uint8_t(pick(0, 3) != 0);
            g_new_budget = budget;
            rc = ddp_set_local_used(r, used.data());
            g_new_budget = -1;
            expect(known_status(rc), "used status", seed, step);
        } else if (op < 97) {                             // regroup
            std::vector<int32_t> firsts;
            for (int b = 0; b < B; ++b)
                if (b == 0 || pick(0, 2) == 0) firsts.push_back(b);
            if (pick(0, 5) == 0 && !firsts.empty()) firsts.back() = B + 3;   // invalid list
            g_new_budget = budget;
            rc = ddp_set_bucket_groups(r, firsts.data(), int32_t(firsts.size()));
            g_new_budget = -1;
            expect(known_status(rc), "groups status", seed, step);
        } else {                                          // introspection
            int64_t nb = 0, off = 0;
            int32_t np = 0, n = 0;
            const int b = pick(-1, B);
            rc = ddp_get_bucket(r, b, &nb, &off, &np);
            expect(known_status(rc) && (rc != DDP_OK || (b >= 0 && b < B)), "get_bucket", seed, step);
            std::vector<int32_t> ro(P);
            ddp_get_ready_order(r, ro.data(), &n);
            expect(n >= 0 && n <= P, "ready order length", seed, step);
        }
        // the callback saw buckets 0, 1, 2, ... of this backward, and nothing after a failure
        for (size_t i = 0; i < rec.seen.size(); ++i)
            expect(rec.seen[i] == int32_t(i), "buckets out of order or repeated", seed, step);
        if (rec.failed)
            expect(rec.seen.back() == rec.fail_at, "a bucket launched after a failed one", seed, step);
        int32_t launched = -1;
        ddp_get_launched(r, &launched);
        expect(launched >= int32_t(rec.seen.size()), "launched count behind the callbacks", seed, step);
    }
    expect(ddp_reducer_destroy(r) == DDP_OK, "destroy", seed, -1);
}

}  // namespace

int main(int argc, char **argv)
{
    const int seeds = argc > 1 ? std::atoi(argv[1]) : 200;
    g_oom = argc > 2 && std::string(argv[2]) == "oom";
    for (int s = 0; s < seeds; ++s) run(s);
    if (g_bad) {
        std::fprintf(stderr, "%d violations\n", g_bad);
        return 1;
    }
    std::printf("host_fuzz ok: %d sequences\n", seeds);
    return 0;
}
