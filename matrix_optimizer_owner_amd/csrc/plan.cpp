// plan.cpp - lowering of an owner table to a step plan.  Host only: this file
// makes no HIP call, so every rule here is testable without a GPU.
//
// The owner table is the MatrixShard-style metadata of "MatrixFSDP:
// Communication-Free Matrix Optimizers Under ZeRO-3 Parameter Sharding"
// (arXiv 2607.05895, Abstract): it carries which whole tensors this owner
// holds and routes each one to its optimizer - 2D weights to Muon, the
// non-matrix tail to AdamW (Abstract), with empty shards legal (Abstract:
// non-owners hold empty shards).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>

#include "plan_internal.h"

namespace mfsdp {

static thread_local std::string g_last_error;

mfsdp_status fail(mfsdp_status status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

void clear_error() { g_last_error.clear(); }

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 22;  // uint16 tile indices at 128-tiles need < 2^23

int elem_bytes(int32_t dtype) { return dtype == kBF16 ? 2 : 4; }

bool finite(float x) { return std::isfinite(x); }

mfsdp_status check_hparams(const mfsdp_hparams& hp) {
    const float fs[] = {hp.lr, hp.weight_decay, hp.momentum, hp.ns_a, hp.ns_b, hp.ns_c, hp.ns_eps,
                        hp.adam_lr, hp.adam_beta1, hp.adam_beta2, hp.adam_eps, hp.adam_weight_decay};
    for (float f : fs)
        if (!finite(f)) return fail(MFSDP_ERR_INVALID_ARGUMENT, "hyper-parameter is not finite");
    if (hp.ns_steps < 0 || hp.ns_steps > 64)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "ns_steps must be in [0, 64]");
    if (hp.ns_eps < 0.f) return fail(MFSDP_ERR_INVALID_ARGUMENT, "ns_eps must be >= 0");
    if (hp.guard_bytes > (1u << 24)) return fail(MFSDP_ERR_INVALID_ARGUMENT, "guard_bytes above 16 MiB");
    if (hp.momentum_dtype != MFSDP_F32 && hp.momentum_dtype != MFSDP_BF16)
        return fail(MFSDP_ERR_UNSUPPORTED, "momentum_dtype must be MFSDP_F32 or MFSDP_BF16");
    if (hp.lr_scale_mode != 0 && hp.lr_scale_mode != 1)
        return fail(MFSDP_ERR_UNSUPPORTED, "lr_scale_mode must be 0 or 1");
    if (hp.ns_precision != 0 && hp.ns_precision != 1)
        return fail(MFSDP_ERR_UNSUPPORTED, "ns_precision must be 0 (bf16) or 1 (fp32)");
    for (int t : {hp.ns_tile_gram, hp.ns_tile_poly, hp.ns_tile_update})
        if (t != 0 && t != kTileSmall && t != kTileLarge)
            return fail(MFSDP_ERR_UNSUPPORTED, "ns_tile_* must be 0 (planner's choice), 128 or 256");
    if (hp.nesterov != 0 && hp.nesterov != 1)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "nesterov must be 0 or 1");
    if (hp.adam_beta1 < 0.f || hp.adam_beta1 >= 1.f || hp.adam_beta2 < 0.f || hp.adam_beta2 >= 1.f)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "adam betas must be in [0, 1)");
    return MFSDP_OK;
}

double shape_scale(int64_t rows, int64_t cols, int mode) {
    if (mode == 0) return std::sqrt(std::max(1.0, double(rows) / double(cols)));
    return 0.2 * std::sqrt(double(std::max(rows, cols)));
}

// Tiles of one matrix for one phase in 2D chunks of cr x cc tiles
// (upper-triangle tiles only for the symmetric phases).  A chunk is what one
// XCD works on at a time, so the operand panels it touches are few and
// shared through that XCD's L2: cr + cc panels for cr * cc = 32 tiles.
// Every phase uses 4 x 8 (for the update, 4 row panels of B and 8 of X^T).
// Against 8 x 4, which counts as many panels per chunk, the mixed 256-matrix
// set's update missed the L2 for 50 GB per launch instead of 67 at the same
// speed, its Gram for 27 GB instead of 29, and the Gram and polynomial ran
// 0.4-1% faster on the three large workloads.
constexpr int kChunk = 32, kXcds = 8;
constexpr int kTriChunkRows = 4, kTriChunkCols = 8, kUpdChunkRows = 4, kUpdChunkCols = 8;
static_assert(kTriChunkRows * kTriChunkCols == kChunk && kUpdChunkRows * kUpdChunkCols == kChunk, "chunk size");

void emit_tiles(std::vector<Tile>& out, uint32_t mat, int tm, int tn, bool upper) {
    const int cr = upper ? kTriChunkRows : kUpdChunkRows, cc = upper ? kTriChunkCols : kUpdChunkCols;
    for (int r0 = 0; r0 < tm; r0 += cr)
        for (int c0 = upper ? (r0 / cc) * cc : 0; c0 < tn; c0 += cc)
            for (int tj = c0; tj < std::min(tn, c0 + cc); ++tj)
                for (int ti = r0; ti < std::min(tm, r0 + cr); ++ti) {
                    if (upper && ti > tj) continue;
                    out.push_back(Tile{mat, uint16_t(ti), uint16_t(tj)});
                }
}

// Reorder a logical tile list (cost-sorted, chunked) into launch order.
// Workgroup w of a launch runs on XCD w % 8; give each XCD whole consecutive
// chunks of kChunk logical tiles: in every round of 8 chunks, chunk k goes to
// XCD k, its tiles at launch indices (round*kChunk + t)*8 + k.  A trailing
// partial round keeps the logical order.
std::vector<Tile> xcd_order(const std::vector<Tile>& logical) {
    const size_t n = logical.size();
    const size_t per_round = size_t(kChunk) * kXcds;
    const size_t full = n / per_round * per_round;
    std::vector<Tile> out(n);
    for (size_t i = 0; i < full; ++i) {
        const size_t round = i / per_round, k = (i % per_round) / kChunk, t = i % kChunk;
        out[(round * kChunk + t) * kXcds + k] = logical[i];
    }
    for (size_t i = full; i < n; ++i) out[i] = logical[i];
    return out;
}

}  // namespace
}  // namespace mfsdp

using namespace mfsdp;

extern "C" mfsdp_status mfsdp_plan_create(const mfsdp_entry* entries, int64_t n, uint64_t param_bytes,
                                          const mfsdp_hparams* hp, mfsdp_plan_t* out) {
    clear_error();
    if (!out) return fail(MFSDP_ERR_INVALID_ARGUMENT, "out is NULL");
    if (!hp) return fail(MFSDP_ERR_INVALID_ARGUMENT, "hparams is NULL");
    if (n < 0) return fail(MFSDP_ERR_INVALID_ARGUMENT, "negative entry count");
    if (n > 0 && !entries) return fail(MFSDP_ERR_INVALID_ARGUMENT, "entries is NULL");
    if (n > (int64_t(1) << 24)) return fail(MFSDP_ERR_UNSUPPORTED, "too many entries");
    if (mfsdp_status st = check_hparams(*hp); st != MFSDP_OK) return st;

    mfsdp_plan_s* plan = new (std::nothrow) mfsdp_plan_s();
    if (!plan) return fail(MFSDP_ERR_INTERNAL, "out of host memory");
    static std::atomic<uint64_t> next_id{1};
    plan->id = next_id.fetch_add(1);
    try {
        plan->entries.assign(entries, entries + n);
        plan->hp = *hp;
        plan->info.resize(size_t(n));

        // ---- per-entry validation and routing ----
        struct Span { uint64_t lo, hi; int64_t idx; };
        std::vector<Span> spans;
        for (int64_t i = 0; i < n; ++i) {
            const mfsdp_entry& e = entries[i];
            if (e.rows < 0 || e.cols < 0) {
                delete plan;
                return fail(MFSDP_ERR_INVALID_ARGUMENT, "entry " + std::to_string(i) + ": negative dimension");
            }
            if (e.dtype != kF32 && e.dtype != kBF16) {
                delete plan;
                return fail(MFSDP_ERR_UNSUPPORTED, "entry " + std::to_string(i) + ": unsupported dtype");
            }
            if (e.role != MFSDP_ROLE_AUTO && e.role != MFSDP_ROLE_MUON && e.role != MFSDP_ROLE_ADAMW) {
                delete plan;
                return fail(MFSDP_ERR_UNSUPPORTED, "entry " + std::to_string(i) + ": unknown role");
            }
            if (e.rows > kMaxDim || e.cols > kMaxDim) {
                delete plan;
                return fail(MFSDP_ERR_UNSUPPORTED, "entry " + std::to_string(i) + ": dimension above 2^22");
            }
            if (e.offset % 16 != 0) {
                delete plan;
                return fail(MFSDP_ERR_MISALIGNED, "entry " + std::to_string(i) + ": offset not 16-byte aligned");
            }
            const uint64_t numel = uint64_t(e.rows) * uint64_t(e.cols);
            const uint64_t bytes = numel * uint64_t(elem_bytes(e.dtype));
            if (e.offset > param_bytes || bytes > param_bytes - e.offset) {
                delete plan;
                return fail(MFSDP_ERR_INVALID_ARGUMENT, "entry " + std::to_string(i) + ": extends past param_bytes");
            }
            mfsdp_entry_info& inf = plan->info[size_t(i)];
            std::memset(&inf, 0, sizeof(inf));
            if (numel == 0) {
                inf.role = -1;
                continue;
            }
            spans.push_back(Span{e.offset, e.offset + bytes, i});
            plan->max_param_end = std::max(plan->max_param_end, e.offset + bytes);
            int role = e.role;
            if (role == MFSDP_ROLE_AUTO) role = (e.rows > 1 && e.cols > 1) ? MFSDP_ROLE_MUON : MFSDP_ROLE_ADAMW;
            inf.role = role;
            if (role == MFSDP_ROLE_MUON) {
                inf.transposed = e.rows > e.cols ? 1 : 0;
                inf.m = std::min(e.rows, e.cols);
                inf.n = std::max(e.rows, e.cols);
                inf.lr_scale = float(shape_scale(e.rows, e.cols, hp->lr_scale_mode));
            }
        }
        std::sort(spans.begin(), spans.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
        for (size_t k = 1; k < spans.size(); ++k)
            if (spans[k].lo < spans[k - 1].hi) {
                const int64_t i = spans[k - 1].idx, j = spans[k].idx;
                delete plan;
                return fail(MFSDP_ERR_OVERLAP,
                            "entries " + std::to_string(i) + " and " + std::to_string(j) + " overlap");
            }

        // ---- state layout: Muon momentum (momentum_dtype), then AdamW moments (fp32) ----
        // every region is followed by `guard` unused bytes (0 unless the
        // caller asked for guard bands)
        const uint64_t guard = align_up(uint64_t(hp->guard_bytes), kAlign);
        const uint64_t mom_bytes = hp->momentum_dtype == MFSDP_BF16 ? 2 : 4;
        uint64_t soff = 0;
        auto state_region = [&](uint64_t bytes, int64_t entry) {
            const uint64_t at = soff;
            plan->regions.push_back(mfsdp_region{at, bytes, MFSDP_BUFFER_STATE, int32_t(entry)});
            soff = align_up(soff + bytes, kAlign) + guard;
            return at;
        };
        for (int64_t i = 0; i < n; ++i) {
            mfsdp_entry_info& inf = plan->info[size_t(i)];
            if (inf.role != MFSDP_ROLE_MUON) continue;
            const uint64_t numel = uint64_t(entries[i].rows) * uint64_t(entries[i].cols);
            inf.state_offset = state_region(numel * mom_bytes, i);
        }
        for (int64_t i = 0; i < n; ++i) {
            mfsdp_entry_info& inf = plan->info[size_t(i)];
            if (inf.role != MFSDP_ROLE_ADAMW) continue;
            const uint64_t numel = uint64_t(entries[i].rows) * uint64_t(entries[i].cols);
            inf.state_offset = state_region(numel * 4, i);
            inf.state_offset2 = state_region(numel * 4, i);
        }
        plan->state_bytes = soff;

        // ---- Muon descriptors, ns_out layout ----
        const int es = hp->ns_precision == 1 ? 4 : 2;
        std::vector<MatDesc> mats;
        std::vector<int32_t> mat_entry;
        uint64_t ns_off = 0;
        for (int64_t i = 0; i < n; ++i) {
            mfsdp_entry_info& inf = plan->info[size_t(i)];
            if (inf.role != MFSDP_ROLE_MUON) continue;
            const mfsdp_entry& e = entries[i];
            MatDesc d;
            std::memset(&d, 0, sizeof(d));
            d.param_off = e.offset;
            d.mom_off = inf.state_offset;
            d.rows = int32_t(e.rows);
            d.cols = int32_t(e.cols);
            d.m = int32_t(inf.m);
            d.n = int32_t(inf.n);
            d.mp = int32_t(align_up(uint64_t(inf.m), kPad));
            d.np = int32_t(align_up(uint64_t(inf.n), kPad));
            // the kernels address one matrix's Newton-Schulz buffers with
            // 32-bit signed byte offsets
            d.ld = d.mp;
            if (uint64_t(d.ld) * uint64_t(d.np) * uint64_t(es) >= (uint64_t(1) << 31)) {
                delete plan;
                return fail(MFSDP_ERR_UNSUPPORTED, "entry " + std::to_string(i) +
                                                       ": padded Newton-Schulz buffer of 2 GiB or more");
            }
            d.transposed = inf.transposed;
            d.dtype = e.dtype;
            // the kernels' step lr * scale, rounded once to fp32
            d.lr_step = float(double(hp->lr) * shape_scale(e.rows, e.cols, hp->lr_scale_mode));
            const int ncols_nat = inf.transposed ? d.mp : d.np;  // padded natural column count
            d.k1_tiles_c = ncols_nat / kK1Tile;
            inf.ns_out_offset = ns_off;
            d.ns_out_off = ns_off;
            ns_off = align_up(ns_off + uint64_t(e.rows) * uint64_t(e.cols), 64);
            mats.push_back(d);
            mat_entry.push_back(int32_t(i));
        }
        plan->ns_out_elems = ns_off;

        std::vector<TailDesc> tails;
        std::vector<int32_t> tail_begin(1, 0);
        for (int64_t i = 0; i < n; ++i) {
            const mfsdp_entry_info& inf = plan->info[size_t(i)];
            if (inf.role != MFSDP_ROLE_ADAMW) continue;
            TailDesc t;
            std::memset(&t, 0, sizeof(t));
            t.param_off = entries[i].offset;
            t.m1_off = inf.state_offset;
            t.m2_off = inf.state_offset2;
            t.numel = entries[i].rows * entries[i].cols;
            t.dtype = entries[i].dtype;
            tails.push_back(t);
            const int64_t chunks = (t.numel + kTailChunk - 1) / kTailChunk;
            tail_begin.push_back(int32_t(tail_begin.back() + chunks));
        }

        // ---- grouped tile lists, longest contraction first ----
        const int nm = int(mats.size());
        std::vector<int> order(static_cast<size_t>(nm));
        for (int k = 0; k < nm; ++k) order[size_t(k)] = k;
        auto by_cost = [&](auto cost) {
            std::vector<int> o = order;
            std::stable_sort(o.begin(), o.end(), [&](int x, int y) { return cost(x) > cost(y); });
            return o;
        };
        // tile edge per phase: 256 when the phase has enough 256-tiles to fill
        // the chip several times over, else 128
        auto count = [&](bool upper, bool full_n, int t) {
            int64_t c = 0;
            for (const MatDesc& d : mats) {
                const int64_t tm = d.mp / t, tn = full_n ? d.np / t : tm;
                c += upper ? tm * (tm + 1) / 2 : tm * tn;
            }
            return c;
        };
        // tile edges forced by the caller (0: the planner's choice)
        const int forced[3] = {hp->ns_tile_gram, hp->ns_tile_poly, hp->ns_tile_update};
        auto pick = [&](int phase, bool upper, bool full_n) {
            if (forced[phase]) return forced[phase];
            return count(upper, full_n, kTileLarge) >= kLargeTileMin ? kTileLarge : kTileSmall;
        };
        const int tg = pick(0, true, false), tp = pick(1, true, false), tu = pick(2, false, true);
        std::vector<Tile> gram, poly, upd;
        for (int k : by_cost([&](int x) { return int64_t(mats[size_t(x)].np); }))
            emit_tiles(gram, uint32_t(k), mats[size_t(k)].mp / tg, mats[size_t(k)].mp / tg, true);
        for (int k : by_cost([&](int x) { return int64_t(mats[size_t(x)].mp); }))
            emit_tiles(poly, uint32_t(k), mats[size_t(k)].mp / tp, mats[size_t(k)].mp / tp, true);
        for (int k : by_cost([&](int x) { return int64_t(mats[size_t(x)].mp); }))
            emit_tiles(upd, uint32_t(k), mats[size_t(k)].mp / tu, mats[size_t(k)].np / tu, false);
        gram = xcd_order(gram);
        poly = xcd_order(poly);
        upd = xcd_order(upd);
        // Wave quantisation of the update: when a 256-tile list would leave a
        // last round of at most kSplitTailMax tiles (one block per CU, so most
        // CUs idle for a whole tile time), those tiles run instead as four
        // 128-tiles each in a second launch (two blocks per CU), which ends in
        // about half a 256-tile time.  Not applied when the tile edge is forced.
        std::vector<Tile> upd_tail;
        if (tu == kTileLarge && !forced[2]) {
            const size_t r = upd.size() % size_t(kCus);
            if (r > 0 && r <= size_t(kSplitTailMax) && upd.size() > r) {
                for (size_t k = upd.size() - r; k < upd.size(); ++k)
                    for (int i = 0; i < 2; ++i)
                        for (int j = 0; j < 2; ++j)
                            upd_tail.push_back(Tile{upd[k].mat, uint16_t(2 * upd[k].ti + i), uint16_t(2 * upd[k].tj + j)});
                upd.resize(upd.size() - r);
            }
        }

        std::vector<int32_t> k1_begin(1, 0);
        for (const MatDesc& d : mats) {
            const int64_t rows_p = d.transposed ? d.np : d.mp;  // padded natural row count
            const int64_t blocks = (rows_p / kK1Tile) * int64_t(d.k1_tiles_c);
            if (k1_begin.back() + blocks > int64_t(INT32_MAX)) {
                delete plan;
                return fail(MFSDP_ERR_UNSUPPORTED, "owner buffer too large for one step");
            }
            k1_begin.push_back(int32_t(k1_begin.back() + blocks));
        }
        if (upd.size() > size_t(INT32_MAX) || tail_begin.back() < 0) {
            delete plan;
            return fail(MFSDP_ERR_UNSUPPORTED, "owner buffer too large for one step");
        }

        // ---- descriptor blob and workspace map ----
        WorkspaceMap& w = plan->map;
        std::memset(&w, 0, sizeof(w));
        uint64_t off = 0;
        auto section = [&](uint64_t bytes) {
            const uint64_t at = off;
            off = align_up(off + bytes, kAlign);
            return at;
        };
        // a region of its own, followed by the guard gap
        auto region = [&](uint64_t bytes, int64_t entry) {
            const uint64_t at = off;
            plan->regions.push_back(mfsdp_region{at, bytes, MFSDP_BUFFER_WORKSPACE, int32_t(entry)});
            off = align_up(off + bytes, kAlign) + guard;
            return at;
        };
        w.off_mat = section(mats.size() * sizeof(MatDesc));
        w.off_k1_begin = section(k1_begin.size() * sizeof(int32_t));
        w.off_gram = section(gram.size() * sizeof(Tile));
        w.off_poly = section(poly.size() * sizeof(Tile));
        w.off_upd = section(upd.size() * sizeof(Tile));
        w.off_upd_tail = section(upd_tail.size() * sizeof(Tile));
        w.off_tail = section(tails.size() * sizeof(TailDesc));
        w.off_tail_begin = section(tail_begin.size() * sizeof(int32_t));
        w.desc_bytes = off;
        // the descriptor blob is uploaded by one copy, so it is one region
        plan->regions.push_back(mfsdp_region{0, off, MFSDP_BUFFER_WORKSPACE, -1});
        off += guard;
        w.off_s = region(mats.size() * sizeof(float), -1);
        w.off_partials = region(uint64_t(k1_begin.back()) * sizeof(float), -1);
        for (size_t k = 0; k < mats.size(); ++k) {
            MatDesc& d = mats[k];
            const uint64_t xbytes = uint64_t(d.ld) * uint64_t(d.np) * uint64_t(es);
            const uint64_t abytes = uint64_t(d.ld) * uint64_t(d.mp) * uint64_t(es);
            d.x_off[0] = region(xbytes, mat_entry[k]);
            d.x_off[1] = region(xbytes, mat_entry[k]);
            d.a_off = region(abytes, mat_entry[k]);
            d.b_off = region(abytes, mat_entry[k]);
        }
        w.total_bytes = off;
        w.n_mat = nm;
        w.n_tail = int32_t(tails.size());
        w.n_gram = int32_t(gram.size());
        w.n_poly = int32_t(poly.size());
        w.n_upd = int32_t(upd.size());
        w.n_upd_tail = int32_t(upd_tail.size());
        w.n_k1_blocks = k1_begin.back();
        w.n_tail_chunks = tail_begin.back();
        w.tile_gram = tg;
        w.tile_poly = tp;
        w.tile_upd = tu;

        plan->desc_blob.assign(size_t(w.desc_bytes), 0);
        auto put = [&](uint64_t at, const void* src, size_t bytes) {
            if (bytes) std::memcpy(plan->desc_blob.data() + at, src, bytes);
        };
        put(w.off_mat, mats.data(), mats.size() * sizeof(MatDesc));
        put(w.off_k1_begin, k1_begin.data(), k1_begin.size() * sizeof(int32_t));
        put(w.off_gram, gram.data(), gram.size() * sizeof(Tile));
        put(w.off_poly, poly.data(), poly.size() * sizeof(Tile));
        put(w.off_upd, upd.data(), upd.size() * sizeof(Tile));
        put(w.off_upd_tail, upd_tail.data(), upd_tail.size() * sizeof(Tile));
        put(w.off_tail, tails.data(), tails.size() * sizeof(TailDesc));
        put(w.off_tail_begin, tail_begin.data(), tail_begin.size() * sizeof(int32_t));
    } catch (const std::bad_alloc&) {
        delete plan;
        return fail(MFSDP_ERR_INTERNAL, "out of host memory");
    } catch (...) {
        delete plan;
        return fail(MFSDP_ERR_INTERNAL, "unexpected exception in plan creation");
    }
    *out = plan;
    return MFSDP_OK;
}

extern "C" mfsdp_status mfsdp_plan_state_bytes(mfsdp_plan_t plan, uint64_t* bytes) {
    clear_error();
    if (!plan || !bytes) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL argument");
    *bytes = plan->state_bytes;
    return MFSDP_OK;
}

extern "C" mfsdp_status mfsdp_plan_workspace_bytes(mfsdp_plan_t plan, uint64_t* bytes) {
    clear_error();
    if (!plan || !bytes) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL argument");
    *bytes = plan->map.total_bytes;
    return MFSDP_OK;
}

extern "C" mfsdp_status mfsdp_plan_ns_out_elems(mfsdp_plan_t plan, uint64_t* elems) {
    clear_error();
    if (!plan || !elems) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL argument");
    *elems = plan->ns_out_elems;
    return MFSDP_OK;
}

extern "C" mfsdp_status mfsdp_plan_num_events(mfsdp_plan_t plan, uint32_t* n) {
    clear_error();
    if (!plan || !n) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL argument");
    *n = uint32_t(3 + 3 * plan->hp.ns_steps);
    return MFSDP_OK;
}

extern "C" mfsdp_status mfsdp_plan_num_entries(mfsdp_plan_t plan, int64_t* n) {
    clear_error();
    if (!plan || !n) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL argument");
    *n = int64_t(plan->entries.size());
    return MFSDP_OK;
}

extern "C" mfsdp_status mfsdp_plan_entry_info(mfsdp_plan_t plan, int64_t i, mfsdp_entry_info* info) {
    clear_error();
    if (!plan || !info) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL argument");
    if (i < 0 || i >= int64_t(plan->entries.size())) return fail(MFSDP_ERR_INVALID_ARGUMENT, "entry index out of range");
    *info = plan->info[size_t(i)];
    return MFSDP_OK;
}

extern "C" mfsdp_status mfsdp_plan_regions(mfsdp_plan_t plan, mfsdp_region* regions, int64_t capacity,
                                           int64_t* count) {
    clear_error();
    if (!plan || !count) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL argument");
    if (capacity < 0 || (capacity > 0 && !regions)) return fail(MFSDP_ERR_INVALID_ARGUMENT, "bad capacity or NULL regions");
    const int64_t n = int64_t(plan->regions.size());
    *count = n;
    for (int64_t k = 0; k < std::min(n, capacity); ++k) regions[k] = plan->regions[size_t(k)];
    return MFSDP_OK;
}

extern "C" mfsdp_status mfsdp_plan_destroy(mfsdp_plan_t plan) {
    clear_error();
    delete plan;
    return MFSDP_OK;
}

extern "C" const char* mfsdp_status_string(mfsdp_status status) {
    switch (status) {
        case MFSDP_OK: return "ok";
        case MFSDP_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MFSDP_ERR_OVERLAP: return "table entries overlap";
        case MFSDP_ERR_MISALIGNED: return "entry offset misaligned";
        case MFSDP_ERR_UNSUPPORTED: return "unsupported";
        case MFSDP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MFSDP_ERR_HIP: return "HIP error";
        case MFSDP_ERR_INTERNAL: return "internal error";
    }
    return "unknown status";
}

extern "C" const char* mfsdp_last_error_message(void) { return g_last_error.c_str(); }
