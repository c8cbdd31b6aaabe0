// layout.h - device descriptor formats and tiling constants shared by the
// host planner (plan.cpp, plain C++) and the HIP kernels.
//
// Workspace map (byte offsets, all 256-byte aligned):
//   [desc]      descriptor blob written by the step from the plan:
//                 MatDesc[n_mat], k1_begin[n_mat+1], Tile gram[], Tile poly[],
//                 Tile upd[], TailDesc[n_tail], tail_begin[n_tail+1]
//   [s]         float[n_mat]: 1/(||U||_F + eps) per Muon matrix
//   [partials]  float[n_k1_blocks]: sum of u^2 over one momentum-kernel tile
//   per matrix: XT0 and XT1 (np x mp, ping-pong), A and B (mp x mp) in the
//               Newton-Schulz storage type (bf16 or fp32), in panel blocks
//               (below); ld = mp columns.
//
// Panel blocks: a Newton-Schulz buffer of R rows and ld columns (R and ld
// multiples of 256) is stored as (R/256) x (ld*es/128) blocks of 256 rows x
// 128 bytes (CB = 128/es columns), each block contiguous (32 KB) with its
// rows at a 128-byte pitch, blocks in row-major order: element (r, c) sits at
// element offset ((r/256) * (ld/CB) + c/CB) * 256*CB + (r%256) * CB + c%CB.
// One stage of a contraction tile (256 or 128 rows x 128 bytes of the
// contraction index) is then one contiguous piece of a block.  With a plain
// row-major layout each of a stage's rows was a separate 128-byte piece at a
// pitch of ld elements: on the mixed 256-matrix set the update's main loop
// then took 2870 shader cycles per stage (2048 of them MFMA), against 2590
// from contiguous pieces.  Its MFMA pipes went from 72% to 75% busy, but
// the power-limited clock fell from 1.63 to 1.56 GHz, so the update gained
// only 1-3% in time.
//
// Orientation: every Muon matrix is handled as X (m x n, m <= n).  A tall
// matrix (rows > cols) is stored transposed.  m and n are padded to
// multiples of kPad with zeros; the zeros stay zero through every
// Newton-Schulz iteration (rows and columns of zeros map to zeros), so the
// contraction kernels need no bounds checks.  X is kept only as X^T
// (n x m): the update reads it along its rows (the contraction index m), the
// Gram reads it K-major through the transposing LDS read.
#pragma once
#include <stdint.h>

namespace mfsdp {

constexpr int kPad = 256;          // padding granule of m and n in the workspace
constexpr int kTileSmall = 128;    // output tile edges of the contraction kernels
constexpr int kTileLarge = 256;
constexpr int kLargeTileMin = 512; // a phase uses 256-tiles when it has at least this many
constexpr int kCus = 256;          // compute units of the part (one 256-tile block each)
constexpr int kSplitTailMax = 64;  // a last update round of at most this many 256-tiles runs as 128-tiles
constexpr int kK1Tile = 128;       // tile edge of the momentum kernel
constexpr int kBlockRows = 256;    // rows of a panel block of the Newton-Schulz buffers
constexpr int kBlockBytes = 128;   // bytes of a panel block's row
constexpr int kTailChunk = 2048;   // elements per AdamW block
constexpr uint64_t kAlign = 256;

enum Dtype : int32_t { kF32 = 0, kBF16 = 1 };

struct MatDesc {
    uint64_t param_off;    // bytes into params and grads
    uint64_t mom_off;      // bytes into state (fp32 momentum, rows x cols)
    uint64_t x_off[2];     // bytes into workspace: X^T ping-pong (np rows of ld, panel blocks)
    int64_t ld;            // columns (elements) of the X^T, A and B buffers: mp
    uint64_t a_off;        // bytes into workspace: A  (mp rows of ld, panel blocks)
    uint64_t b_off;        // bytes into workspace: B  (mp rows of ld, panel blocks)
    uint64_t ns_out_off;   // element offset into ns_out (fp32, rows x cols)
    int32_t rows, cols;    // shape as given
    int32_t m, n;          // oriented, m <= n
    int32_t mp, np;        // padded to kPad
    int32_t transposed;    // rows > cols
    int32_t dtype;         // param / grad storage type
    float lr_step;         // lr * shape scale of the learning rate, rounded once to fp32
    int32_t k1_tiles_c;    // momentum-kernel tile columns (natural layout)
};

// One output tile of a grouped contraction: matrix index and tile coordinates
// in units of the phase's tile edge.
struct Tile {
    uint32_t mat;
    uint16_t ti, tj;
};

struct TailDesc {
    uint64_t param_off;    // bytes into params and grads
    uint64_t m1_off;       // bytes into state (fp32)
    uint64_t m2_off;       // bytes into state (fp32)
    int64_t numel;
    int32_t dtype;
    int32_t pad_;
};

static_assert(sizeof(MatDesc) == 8 * 8 + 4 * 10, "MatDesc layout");
static_assert(sizeof(Tile) == 8, "Tile layout");
static_assert(sizeof(TailDesc) == 40, "TailDesc layout");

// Byte offsets of the sections of the descriptor blob and of the fixed
// workspace regions, plus element counts; filled by the planner.
struct WorkspaceMap {
    uint64_t desc_bytes;
    uint64_t off_mat, off_k1_begin, off_gram, off_poly, off_upd, off_upd_tail, off_tail, off_tail_begin;
    uint64_t off_s, off_partials;
    uint64_t total_bytes;
    int32_t n_mat, n_tail;
    int32_t n_gram, n_poly, n_upd;
    int32_t n_upd_tail;                      // 128-tiles run after the 256-tile update list (see the planner)
    int32_t n_k1_blocks, n_tail_chunks;
    int32_t tile_gram, tile_poly, tile_upd;  // tile edge of each contraction phase
};

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

}  // namespace mfsdp
