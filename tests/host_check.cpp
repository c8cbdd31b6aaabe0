// host_check.cpp - host-only driver of the owner planner and the checkpoint
// copies (built with g++ against owner_planner.cpp, checkpoint.cpp and
// plan.cpp; no HIP), for runs under host sanitizers.  For seeded random
// tensor lists and owner counts: partition, build every owner's plan from
// its table, scatter random bytes from whole-tensor buffers into the
// owners' flat buffers and gather them back; the bytes must round-trip.
// Also calls each entry point with invalid arguments.  Prints "OK <n>" or
// the first failure; returns non-zero on a failure.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "mfsdp.h"

static int fails = 0;
#define EXPECT(c, ...)                          \
    do {                                        \
        if (!(c)) {                             \
            std::printf("FAIL %s: ", #c);       \
            std::printf(__VA_ARGS__);           \
            std::printf("\n");                  \
            return 1;                           \
        }                                       \
    } while (0)

int main() {
    std::mt19937_64 rng(7);
    int cases = 0;
    for (int trial = 0; trial < 40; ++trial) {
        const int n = 1 + int(rng() % 24), owners = 1 + int(rng() % 6), mdt = int(rng() % 2);
        std::vector<mfsdp_tensor> ts(static_cast<size_t>(n));
        for (auto& t : ts) {
            const int kind = int(rng() % 5);
            t.rows = kind == 0 ? 1 : kind == 1 ? 0 : 1 + int64_t(rng() % 700);
            t.cols = 1 + int64_t(rng() % 900);
            t.dtype = rng() % 2 ? MFSDP_BF16 : MFSDP_F32;
            t.role = MFSDP_ROLE_AUTO;
        }
        mfsdp_partition_params pp;
        std::memset(&pp, 0, sizeof(pp));
        pp.n_owners = owners;
        pp.ns_steps = 5;
        pp.momentum_dtype = mdt ? MFSDP_BF16 : MFSDP_F32;
        pp.flop_rate = 1.6e15;
        pp.byte_rate = 5.2e12;
        std::vector<mfsdp_tensor_place> place(static_cast<size_t>(n));
        std::vector<double> cost(static_cast<size_t>(owners));
        std::vector<uint64_t> mem(static_cast<size_t>(owners)), pbytes(static_cast<size_t>(owners));
        EXPECT(mfsdp_owner_partition(ts.data(), n, &pp, place.data(), cost.data(), mem.data(), pbytes.data()) ==
                   MFSDP_OK, "trial %d partition", trial);
        mfsdp_hparams hp;
        std::memset(&hp, 0, sizeof(hp));
        hp.lr = 0.02f; hp.weight_decay = 0.01f; hp.momentum = 0.95f; hp.nesterov = 1; hp.ns_steps = 5;
        hp.ns_a = 3.4445f; hp.ns_b = -4.775f; hp.ns_c = 2.0315f; hp.ns_eps = 1e-7f;
        hp.adam_lr = 0.02f; hp.adam_beta1 = 0.9f; hp.adam_beta2 = 0.95f; hp.adam_eps = 1e-8f;
        hp.adam_weight_decay = 0.01f; hp.momentum_dtype = pp.momentum_dtype;
        for (int o = 0; o < owners; ++o) {
            std::vector<mfsdp_entry> es;
            std::vector<int> idx;
            for (int i = 0; i < n; ++i)
                if (place[size_t(i)].owner == o) {
                    mfsdp_entry e;
                    e.offset = place[size_t(i)].offset;
                    e.rows = ts[size_t(i)].rows;
                    e.cols = ts[size_t(i)].cols;
                    e.dtype = ts[size_t(i)].dtype;
                    e.role = place[size_t(i)].role;
                    es.push_back(e);
                    idx.push_back(i);
                }
            mfsdp_plan_t plan = nullptr;
            EXPECT(mfsdp_plan_create(es.data(), int64_t(es.size()), pbytes[size_t(o)], &hp, &plan) == MFSDP_OK,
                   "trial %d owner %d plan", trial, o);
            uint64_t sbytes = 0;
            EXPECT(mfsdp_plan_state_bytes(plan, &sbytes) == MFSDP_OK, "state bytes");
            // whole-tensor buffers of random bytes
            const size_t k = es.size();
            std::vector<std::vector<uint8_t>> t0(k), s1(k), s2(k), t1(k), r1(k), r2(k);
            std::vector<void*> pt(k), p1(k), p2(k), qt(k), q1(k), q2(k);
            for (size_t j = 0; j < k; ++j) {
                const uint64_t numel = uint64_t(es[j].rows) * uint64_t(es[j].cols);
                mfsdp_entry_info inf;
                EXPECT(mfsdp_plan_entry_info(plan, int64_t(j), &inf) == MFSDP_OK, "info");
                const uint64_t eb = es[j].dtype == MFSDP_BF16 ? 2 : 4;
                const uint64_t mb = inf.role == MFSDP_ROLE_MUON && mdt ? 2 : 4;
                t0[j].resize(numel * eb);
                s1[j].resize(numel * mb);
                s2[j].resize(inf.role == MFSDP_ROLE_ADAMW ? numel * 4 : 0);
                for (auto* v : {&t0[j], &s1[j], &s2[j]})
                    for (auto& b : *v) b = uint8_t(rng());
                t1[j].assign(t0[j].size(), 0);
                r1[j].assign(s1[j].size(), 0);
                r2[j].assign(s2[j].size(), 0);
                pt[j] = t0[j].empty() ? nullptr : t0[j].data();
                p1[j] = s1[j].empty() ? nullptr : s1[j].data();
                p2[j] = s2[j].empty() ? nullptr : s2[j].data();
                qt[j] = t1[j].empty() ? nullptr : t1[j].data();
                q1[j] = r1[j].empty() ? nullptr : r1[j].data();
                q2[j] = r2[j].empty() ? nullptr : r2[j].data();
            }
            std::vector<uint8_t> params(std::max<uint64_t>(pbytes[size_t(o)], 1)), state(std::max<uint64_t>(sbytes, 1));
            EXPECT(mfsdp_owner_scatter(plan, pt.data(), p1.data(), p2.data(), params.data(), params.size(),
                                       state.data(), state.size()) == MFSDP_OK,
                   "trial %d owner %d scatter", trial, o);
            EXPECT(mfsdp_owner_gather(plan, params.data(), params.size(), state.data(), state.size(), qt.data(),
                                      q1.data(), q2.data()) == MFSDP_OK,
                   "trial %d owner %d gather", trial, o);
            for (size_t j = 0; j < k; ++j)
                EXPECT(t0[j] == t1[j] && s1[j] == r1[j] && s2[j] == r2[j], "trial %d owner %d entry %zu", trial, o, j);
            // invalid arguments: a buffer too small, a NULL plan
            if (sbytes > 0)
                EXPECT(mfsdp_owner_gather(plan, params.data(), params.size(), state.data(), sbytes - 1, nullptr,
                                          q1.data(), nullptr) != MFSDP_OK, "short state accepted");
            EXPECT(mfsdp_owner_gather(nullptr, params.data(), params.size(), nullptr, 0, nullptr, nullptr, nullptr) !=
                       MFSDP_OK, "null plan accepted");
            mfsdp_plan_destroy(plan);
            ++cases;
        }
    }
    mfsdp_partition_params bad;
    std::memset(&bad, 0, sizeof(bad));
    EXPECT(mfsdp_owner_partition(nullptr, 1, &bad, nullptr, nullptr, nullptr, nullptr) != MFSDP_OK, "null tensors");
    std::printf("OK %d\n", cases);
    return fails;
}
