// owner_planner.cpp - the balance-aware owner planner: which owner holds
// each whole tensor.  Host only (no HIP call).
//
// "MatrixFSDP: Communication-Free Matrix Optimizers Under ZeRO-3 Parameter
// Sharding" (arXiv 2607.05895), Abstract: one data-parallel rank owns each
// whole 2D weight, tensors that are not matrices are grouped onto a few
// tail owners, and a balance-aware owner planner makes that placement.  The pages give no
// algorithm; the cost and memory model and the objective are stated in
// mfsdp.h (mfsdp_owner_partition).  The memory model follows the layout
// mfsdp_plan_create gives an owner's table.
#include <algorithm>
#include <cmath>
#include <numeric>
#include <string>
#include <vector>

#include "plan_internal.h"

namespace mfsdp {
namespace {

constexpr int64_t kMaxDim = int64_t(1) << 22;  // the plan's dimension limit

struct Item {
    int64_t idx;
    int role;
    double cost;
    uint64_t mem;
    uint64_t bytes;  // parameter bytes
};

uint64_t region(uint64_t bytes) { return align_up(bytes, kAlign); }

}  // namespace
}  // namespace mfsdp

using namespace mfsdp;

extern "C" mfsdp_status mfsdp_owner_partition(const mfsdp_tensor* tensors, int64_t n, const mfsdp_partition_params* pp,
                                              mfsdp_tensor_place* place, double* owner_cost,
                                              uint64_t* owner_mem_bytes, uint64_t* owner_param_bytes) {
    try {
        clear_error();
        if (!pp || n < 0 || (n > 0 && (!tensors || !place)))
            return fail(MFSDP_ERR_INVALID_ARGUMENT, "null pointer or n < 0");
        const int P = pp->n_owners;
        if (P < 1) return fail(MFSDP_ERR_INVALID_ARGUMENT, "n_owners must be >= 1");
        if (pp->ns_steps < 0) return fail(MFSDP_ERR_INVALID_ARGUMENT, "ns_steps must be >= 0");
        if (pp->ns_precision != 0 && pp->ns_precision != 1)
            return fail(MFSDP_ERR_UNSUPPORTED, "ns_precision must be 0 (bf16) or 1 (fp32)");
        if (!(std::isfinite(pp->flop_rate) && pp->flop_rate > 0 && std::isfinite(pp->byte_rate) && pp->byte_rate > 0))
            return fail(MFSDP_ERR_INVALID_ARGUMENT, "flop_rate and byte_rate must be positive and finite");
        if (pp->momentum_dtype != MFSDP_F32 && pp->momentum_dtype != MFSDP_BF16)
            return fail(MFSDP_ERR_UNSUPPORTED, "momentum_dtype must be MFSDP_F32 or MFSDP_BF16");
        const uint64_t cap = pp->mem_cap_bytes;
        const int es_ns = pp->ns_precision == 1 ? 4 : 2;
        const uint64_t es_mom = pp->momentum_dtype == MFSDP_BF16 ? 2 : 4;

        // ---- per-tensor role, cost and memory ----
        std::vector<Item> items(static_cast<size_t>(n));
        for (int64_t i = 0; i < n; ++i) {
            const mfsdp_tensor& t = tensors[i];
            Item& it = items[size_t(i)];
            it.idx = i;
            if (t.rows < 0 || t.cols < 0)
                return fail(MFSDP_ERR_INVALID_ARGUMENT, "tensor " + std::to_string(i) + ": negative dimension");
            if (t.dtype != kF32 && t.dtype != kBF16)
                return fail(MFSDP_ERR_UNSUPPORTED, "tensor " + std::to_string(i) + ": unsupported dtype");
            if (t.role != MFSDP_ROLE_AUTO && t.role != MFSDP_ROLE_MUON && t.role != MFSDP_ROLE_ADAMW)
                return fail(MFSDP_ERR_UNSUPPORTED, "tensor " + std::to_string(i) + ": unknown role");
            if (t.rows > kMaxDim || t.cols > kMaxDim)
                return fail(MFSDP_ERR_UNSUPPORTED, "tensor " + std::to_string(i) + ": dimension above 2^22");
            const uint64_t numel = uint64_t(t.rows) * uint64_t(t.cols);
            const uint64_t es = t.dtype == kBF16 ? 2 : 4;
            int role = t.role == MFSDP_ROLE_AUTO ? ((t.rows > 1 && t.cols > 1) ? MFSDP_ROLE_MUON : MFSDP_ROLE_ADAMW)
                                                 : t.role;
            if (numel == 0) role = MFSDP_ROLE_ADAMW;
            it.role = role;
            it.bytes = numel * es;
            if (role == MFSDP_ROLE_MUON) {
                const double m = double(std::min(t.rows, t.cols)), nn = double(std::max(t.rows, t.cols));
                const uint64_t mp = align_up(uint64_t(std::min(t.rows, t.cols)), kPad);
                const uint64_t np = align_up(uint64_t(std::max(t.rows, t.cols)), kPad);
                const uint64_t ld = mp;
                if (ld * np * uint64_t(es_ns) >= (uint64_t(1) << 31))
                    return fail(MFSDP_ERR_UNSUPPORTED,
                                "tensor " + std::to_string(i) + ": padded Newton-Schulz buffer of 2 GiB or more");
                it.cost = double(pp->ns_steps) * (4.0 * m * m * nn + 2.0 * m * m * m) / pp->flop_rate +
                          double(numel) * double(3 * es + 2 * es_mom + uint64_t(es_ns)) / pp->byte_rate;
                it.mem = 2 * region(numel * es) + region(numel * es_mom) + 2 * region(ld * np * uint64_t(es_ns)) +
                         2 * region(ld * mp * uint64_t(es_ns));
            } else {
                it.cost = double(numel) * double(3 * es + 16) / pp->byte_rate;
                it.mem = 2 * region(numel * es) + 2 * region(numel * 4);
            }
            if (cap && it.mem > cap)
                return fail(MFSDP_ERR_UNSUPPORTED, "tensor " + std::to_string(i) + " alone exceeds the memory cap");
        }

        // ---- longest-processing-time pass ----
        std::vector<int64_t> order(static_cast<size_t>(n));
        std::iota(order.begin(), order.end(), int64_t(0));
        std::stable_sort(order.begin(), order.end(), [&](int64_t x, int64_t y) {
            const Item& a = items[size_t(x)];
            const Item& b = items[size_t(y)];
            if (a.cost != b.cost) return a.cost > b.cost;
            if (a.mem != b.mem) return a.mem > b.mem;
            return x < y;
        });
        std::vector<int> owner(static_cast<size_t>(n), -1);
        std::vector<double> load(size_t(P), 0.0);
        std::vector<uint64_t> mem(size_t(P), 0);
        auto fits = [&](int o, uint64_t extra) { return !cap || mem[size_t(o)] + extra <= cap; };
        for (int64_t k : order) {
            const Item& it = items[size_t(k)];
            int best = -1;
            for (int o = 0; o < P; ++o)
                if (fits(o, it.mem) && (best < 0 || load[size_t(o)] < load[size_t(best)])) best = o;
            if (best < 0)
                return fail(MFSDP_ERR_UNSUPPORTED,
                            "tensor " + std::to_string(k) + ": no owner has room left under the memory cap");
            owner[size_t(k)] = best;
            load[size_t(best)] += it.cost;
            mem[size_t(best)] += it.mem;
        }

        // ---- moves and swaps off the most loaded owner ----
        // Each accepted change lowers the most loaded owner's cost without
        // raising any other owner to or above it, so the largest cost never
        // rises; the bound on rounds only guards against float ties.
        const int64_t max_rounds = 64 * (n + P);
        for (int64_t round = 0; round < max_rounds; ++round) {
            int top = 0;
            for (int o = 1; o < P; ++o)
                if (load[size_t(o)] > load[size_t(top)]) top = o;
            const double L = load[size_t(top)];
            double best_new = L;  // the larger of the two changed owners' costs after the change
            int64_t bt = -1, bu = -1;
            int bo = -1;
            for (int64_t t = 0; t < n; ++t) {
                if (owner[size_t(t)] != top) continue;
                const Item& a = items[size_t(t)];
                if (a.cost <= 0) continue;
                for (int o = 0; o < P; ++o) {
                    if (o == top) continue;
                    // move t to o
                    if (fits(o, a.mem)) {
                        const double nw = std::max(L - a.cost, load[size_t(o)] + a.cost);
                        if (nw < best_new) {
                            best_new = nw;
                            bt = t;
                            bu = -1;
                            bo = o;
                        }
                    }
                    // swap t with a cheaper u on o
                    for (int64_t u = 0; u < n; ++u) {
                        if (owner[size_t(u)] != o) continue;
                        const Item& b = items[size_t(u)];
                        if (b.cost >= a.cost) continue;
                        if (cap && (mem[size_t(o)] - b.mem + a.mem > cap || mem[size_t(top)] - a.mem + b.mem > cap))
                            continue;
                        const double nw = std::max(L - a.cost + b.cost, load[size_t(o)] + a.cost - b.cost);
                        if (nw < best_new) {
                            best_new = nw;
                            bt = t;
                            bu = u;
                            bo = o;
                        }
                    }
                }
            }
            if (bt < 0 || !(best_new < L * (1.0 - 1e-12))) break;
            const Item& a = items[size_t(bt)];
            owner[size_t(bt)] = bo;
            load[size_t(top)] -= a.cost;
            load[size_t(bo)] += a.cost;
            mem[size_t(top)] -= a.mem;
            mem[size_t(bo)] += a.mem;
            if (bu >= 0) {
                const Item& b = items[size_t(bu)];
                owner[size_t(bu)] = top;
                load[size_t(bo)] -= b.cost;
                load[size_t(top)] += b.cost;
                mem[size_t(bo)] -= b.mem;
                mem[size_t(top)] += b.mem;
            }
        }

        // ---- each owner's flat buffer: its tensors in input order ----
        std::vector<uint64_t> end(size_t(P), 0);
        std::vector<double> cost_sum(size_t(P), 0.0);
        std::vector<uint64_t> mem_sum(size_t(P), 0);
        for (int64_t i = 0; i < n; ++i) {
            const Item& it = items[size_t(i)];
            const int o = owner[size_t(i)];
            mfsdp_tensor_place& pl = place[i];
            pl.owner = o;
            pl.role = it.role;
            pl.offset = end[size_t(o)];
            pl.cost = it.cost;
            pl.mem_bytes = it.mem;
            end[size_t(o)] = align_up(end[size_t(o)] + it.bytes, kAlign);
            cost_sum[size_t(o)] += it.cost;  // summed in input order (reproducible)
            mem_sum[size_t(o)] += it.mem;
        }
        for (int o = 0; o < P; ++o) {
            if (owner_cost) owner_cost[o] = cost_sum[size_t(o)];
            if (owner_mem_bytes) owner_mem_bytes[o] = mem_sum[size_t(o)];
            if (owner_param_bytes) owner_param_bytes[o] = end[size_t(o)];
        }
        return MFSDP_OK;
    } catch (const std::bad_alloc&) {
        return fail(MFSDP_ERR_INTERNAL, "out of host memory");
    } catch (...) {
        return fail(MFSDP_ERR_INTERNAL, "unexpected host exception");
    }
}
