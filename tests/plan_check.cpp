// plan_check.cpp - host-only checker of the planner's lowered plan (built
// with g++ against plan.cpp; no HIP).  Reads a table from stdin:
//   ns_precision n
//   offset rows cols dtype role      (n lines)
// and checks the descriptor blob and layout invariants.  Optional arguments
// G P U force the tile edges of the Gram, polynomial and update (the plan's
// ns_tile_* options; 0 = the planner's choice).  Prints "OK <stats>" or the
// first violation, and returns non-zero on a violation.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <set>
#include <tuple>
#include <vector>

#include "plan_internal.h"

using namespace mfsdp;

static int fail_count = 0;
#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            std::printf("FAIL %s: ", #cond);      \
            std::printf(__VA_ARGS__);             \
            std::printf("\n");                    \
            if (++fail_count > 10) return 1;      \
        }                                         \
    } while (0)

int main(int argc, char** argv) {
    int prec = 0;
    long long n = 0;
    if (std::scanf("%d %lld", &prec, &n) != 2) return 2;
    std::vector<mfsdp_entry> es(static_cast<size_t>(n));
    uint64_t pbytes = 0;
    for (auto& e : es) {
        unsigned long long off;
        long long r, c;
        int dt, role;
        if (std::scanf("%llu %lld %lld %d %d", &off, &r, &c, &dt, &role) != 5) return 2;
        e.offset = off;
        e.rows = r;
        e.cols = c;
        e.dtype = dt;
        e.role = role;
        pbytes = std::max<uint64_t>(pbytes, off + uint64_t(r * c) * (dt == 1 ? 2 : 4));
    }
    mfsdp_hparams hp;
    std::memset(&hp, 0, sizeof(hp));
    hp.lr = 0.02f; hp.weight_decay = 0.01f; hp.momentum = 0.95f; hp.nesterov = 1; hp.ns_steps = 5;
    hp.ns_a = 3.4445f; hp.ns_b = -4.775f; hp.ns_c = 2.0315f; hp.ns_eps = 1e-7f; hp.ns_precision = prec;
    hp.adam_lr = 0.02f; hp.adam_beta1 = 0.9f; hp.adam_beta2 = 0.95f; hp.adam_eps = 1e-8f; hp.adam_weight_decay = 0.01f;
    if (argc >= 4) {
        hp.ns_tile_gram = std::atoi(argv[1]);
        hp.ns_tile_poly = std::atoi(argv[2]);
        hp.ns_tile_update = std::atoi(argv[3]);
    }
    mfsdp_plan_t plan = nullptr;
    const mfsdp_status st = mfsdp_plan_create(es.data(), n, pbytes, &hp, &plan);
    CHECK(st == MFSDP_OK, "plan_create failed: %s", mfsdp_last_error_message());
    if (st != MFSDP_OK) return 1;
    const WorkspaceMap& w = plan->map;
    const uint8_t* blob = plan->desc_blob.data();
    const MatDesc* mats = reinterpret_cast<const MatDesc*>(blob + w.off_mat);
    const int es_ns = prec == 1 ? 4 : 2;

    // --- matrices: routing, orientation, padding, scale ---
    int mi = 0;
    for (long long i = 0; i < n; ++i) {
        const mfsdp_entry& e = es[size_t(i)];
        const mfsdp_entry_info& inf = plan->info[size_t(i)];
        if (inf.role != MFSDP_ROLE_MUON) continue;
        const MatDesc& d = mats[mi++];
        CHECK(d.param_off == e.offset, "entry %lld offset", i);
        CHECK(d.rows == e.rows && d.cols == e.cols, "entry %lld shape", i);
        CHECK(d.m == std::min(e.rows, e.cols) && d.n == std::max(e.rows, e.cols), "entry %lld orientation", i);
        CHECK(d.transposed == (e.rows > e.cols ? 1 : 0), "entry %lld transposed flag", i);
        CHECK(d.mp % kPad == 0 && d.np % kPad == 0 && d.mp >= d.m && d.np >= d.n && d.mp - d.m < kPad &&
                  d.np - d.n < kPad, "entry %lld padding", i);
        const double want = std::sqrt(std::max(1.0, double(e.rows) / double(e.cols)));
        CHECK(d.lr_step == float(double(hp.lr) * want), "entry %lld lr step %g vs %g", i, d.lr_step, double(hp.lr) * want);
        CHECK(d.mom_off == inf.state_offset && d.mom_off % kAlign == 0, "entry %lld momentum offset", i);
    }
    CHECK(mi == w.n_mat, "matrix count %d vs %d", mi, w.n_mat);

    // --- workspace regions: aligned, disjoint, inside the total ---
    std::vector<std::pair<uint64_t, uint64_t>> regs;
    regs.push_back({0, w.desc_bytes});
    regs.push_back({w.off_s, uint64_t(w.n_mat) * 4});
    regs.push_back({w.off_partials, uint64_t(w.n_k1_blocks) * 4});
    for (int k = 0; k < w.n_mat; ++k) {
        const MatDesc& d = mats[k];
        CHECK(d.ld == d.mp && d.mp % kBlockRows == 0 && d.np % kBlockRows == 0 && (d.ld * es_ns) % kBlockBytes == 0, "matrix %d panel blocks", k);
        const uint64_t xb = uint64_t(d.ld) * d.np * es_ns, ab = uint64_t(d.ld) * d.mp * es_ns;
        regs.push_back({d.x_off[0], xb});
        regs.push_back({d.x_off[1], xb});
        regs.push_back({d.a_off, ab});
        regs.push_back({d.b_off, ab});
    }
    std::sort(regs.begin(), regs.end());
    for (size_t k = 0; k < regs.size(); ++k) {
        CHECK(regs[k].first % kAlign == 0, "region %zu misaligned", k);
        CHECK(regs[k].first + regs[k].second <= w.total_bytes, "region %zu past the end", k);
        if (k) CHECK(regs[k - 1].first + regs[k - 1].second <= regs[k].first, "regions %zu/%zu overlap", k - 1, k);
    }

    // --- momentum-kernel block prefix ---
    const int32_t* k1 = reinterpret_cast<const int32_t*>(blob + w.off_k1_begin);
    CHECK(k1[0] == 0, "k1 prefix start");
    for (int k = 0; k < w.n_mat; ++k) {
        const MatDesc& d = mats[k];
        const int rows_p = d.transposed ? d.np : d.mp, cols_p = d.transposed ? d.mp : d.np;
        CHECK(d.k1_tiles_c == cols_p / kK1Tile, "matrix %d k1 columns", k);
        CHECK(k1[k + 1] - k1[k] == (rows_p / kK1Tile) * (cols_p / kK1Tile), "matrix %d k1 blocks", k);
    }
    CHECK(k1[w.n_mat] == w.n_k1_blocks, "k1 total");

    // --- tile lists: every tile of every matrix exactly once ---
    auto check_tiles = [&](uint64_t off, int count, int tile, bool upper, bool full_n, const char* name) {
        const Tile* t = reinterpret_cast<const Tile*>(blob + off);
        std::set<std::tuple<uint32_t, int, int>> seen;
        size_t expect = 0;
        for (int k = 0; k < w.n_mat; ++k) {
            const int tm = mats[k].mp / tile, tn = full_n ? mats[k].np / tile : tm;
            expect += upper ? size_t(tm) * (tm + 1) / 2 : size_t(tm) * tn;
        }
        if (size_t(count) != expect) {
            std::printf("FAIL %s: %d tiles, expected %zu\n", name, count, expect);
            ++fail_count;
            return;
        }
        for (int k = 0; k < count; ++k) {
            const int tm = mats[t[k].mat].mp / tile, tn = full_n ? mats[t[k].mat].np / tile : tm;
            if (t[k].mat >= uint32_t(w.n_mat) || t[k].ti >= tm || t[k].tj >= tn || (upper && t[k].ti > t[k].tj)) {
                std::printf("FAIL %s: tile %d out of range\n", name, k);
                ++fail_count;
                return;
            }
            if (!seen.insert({t[k].mat, t[k].ti, t[k].tj}).second) {
                std::printf("FAIL %s: tile %d repeated\n", name, k);
                ++fail_count;
                return;
            }
        }
    };
    check_tiles(w.off_gram, w.n_gram, w.tile_gram, true, false, "gram");
    check_tiles(w.off_poly, w.n_poly, w.tile_poly, true, false, "poly");
    if (w.n_upd_tail == 0) {
        check_tiles(w.off_upd, w.n_upd, w.tile_upd, false, true, "update");
    } else {
        // a 256-tile list plus a 128-tile remainder: together every 128-cell once
        CHECK(w.tile_upd == 256 && w.n_upd % 256 == 0 && w.n_upd_tail % 4 == 0 && w.n_upd_tail <= 4 * 64,
              "update split shape %d + %d", w.n_upd, w.n_upd_tail);
        std::set<std::tuple<uint32_t, int, int>> cells;
        size_t expect = 0, got = 0;
        for (int k = 0; k < w.n_mat; ++k) expect += size_t(mats[k].mp / 128) * (mats[k].np / 128);
        const Tile* t = reinterpret_cast<const Tile*>(blob + w.off_upd);
        for (int k = 0; k < w.n_upd; ++k)
            for (int i = 0; i < 2; ++i)
                for (int j = 0; j < 2; ++j) {
                    CHECK(t[k].mat < uint32_t(w.n_mat) && t[k].ti < mats[t[k].mat].mp / 256 && t[k].tj < mats[t[k].mat].np / 256,
                          "update tile %d out of range", k);
                    got += cells.insert({t[k].mat, 2 * t[k].ti + i, 2 * t[k].tj + j}).second;
                }
        const Tile* u = reinterpret_cast<const Tile*>(blob + w.off_upd_tail);
        for (int k = 0; k < w.n_upd_tail; ++k) {
            CHECK(u[k].mat < uint32_t(w.n_mat) && u[k].ti < mats[u[k].mat].mp / 128 && u[k].tj < mats[u[k].mat].np / 128,
                  "update tail tile %d out of range", k);
            got += cells.insert({u[k].mat, u[k].ti, u[k].tj}).second;
        }
        CHECK(got == size_t(w.n_upd) * 4 + size_t(w.n_upd_tail) && got == expect, "update cells %zu of %zu", got, expect);
    }
    CHECK(w.tile_gram == 128 || w.tile_gram == 256, "gram tile edge");
    CHECK(w.tile_upd == 128 || w.tile_upd == 256, "update tile edge");

    // --- state layout and AdamW chunks ---
    std::vector<std::pair<uint64_t, uint64_t>> sregs;
    const TailDesc* tails = reinterpret_cast<const TailDesc*>(blob + w.off_tail);
    const int32_t* tb = reinterpret_cast<const int32_t*>(blob + w.off_tail_begin);
    int ti = 0;
    for (long long i = 0; i < n; ++i) {
        const mfsdp_entry& e = es[size_t(i)];
        const mfsdp_entry_info& inf = plan->info[size_t(i)];
        const uint64_t bytes = uint64_t(e.rows * e.cols) * 4;
        if (inf.role == MFSDP_ROLE_MUON) sregs.push_back({inf.state_offset, bytes});
        if (inf.role == MFSDP_ROLE_ADAMW) {
            sregs.push_back({inf.state_offset, bytes});
            sregs.push_back({inf.state_offset2, bytes});
            const TailDesc& t = tails[ti];
            CHECK(t.param_off == e.offset && t.numel == e.rows * e.cols && t.dtype == e.dtype, "tail %d", ti);
            CHECK(t.m1_off == inf.state_offset && t.m2_off == inf.state_offset2, "tail %d state", ti);
            CHECK(tb[ti + 1] - tb[ti] == int32_t((t.numel + kTailChunk - 1) / kTailChunk), "tail %d chunks", ti);
            ++ti;
        }
    }
    CHECK(ti == w.n_tail, "tail count");
    std::sort(sregs.begin(), sregs.end());
    for (size_t k = 0; k < sregs.size(); ++k) {
        CHECK(sregs[k].first % kAlign == 0, "state region %zu misaligned", k);
        CHECK(sregs[k].first + sregs[k].second <= plan->state_bytes, "state region %zu past the end", k);
        if (k) CHECK(sregs[k - 1].first + sregs[k - 1].second <= sregs[k].first, "state regions overlap");
    }
    if (!fail_count)
        std::printf("OK mats=%d tails=%d gram=%d poly=%d upd=%d+%d tiles=%d/%d/%d ws=%llu state=%llu\n", w.n_mat,
                    w.n_tail, w.n_gram, w.n_poly, w.n_upd, w.n_upd_tail, w.tile_gram, w.tile_poly, w.tile_upd,
                    (unsigned long long)w.total_bytes, (unsigned long long)plan->state_bytes);
    mfsdp_plan_destroy(plan);
    return fail_count ? 1 : 0;
}
