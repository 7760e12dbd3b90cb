// Destination bins of the core backward's grad_x samples, shared by the count pass,
// the record pass and the LDS-tiled gradient kernel (included inside namespace dcn's
// anonymous namespace by each, after dcn_common.hpp). A sample whose bilinear cell
// has top-left corner (y0, x0) belongs to the 16x16 input tile holding (y0+1, x0+1),
// with a sub-bin for cells on that tile's first row and/or column. P supplies the
// image size H, W, groups G and bin grid TY, TX (and sh, sw, ph, pw for windows).
#pragma once

constexpr int kBinTile = 16;

// Home bin of a sample whose bilinear cell has top-left corner (y0, x0); false
// when no corner of the cell is inside the image. The home tile holds the corner
// (y0+1, x0+1); `local` packs the cell's position in that tile (4 bits each).
template <class P>
__device__ __forceinline__ bool home_bin(int y0, int x0, int n, int g, const P &p,
                                         unsigned &bin, unsigned &local) {
    if (y0 < -1 || y0 > p.H - 1 || x0 < -1 || x0 > p.W - 1) return false;
    const int ty = (y0 + 1) / kBinTile, tx = (x0 + 1) / kBinTile;
    const int ly = y0 + 1 - ty * kBinTile, lx = x0 + 1 - tx * kBinTile;
    const unsigned sub = (ly == 0 ? 1u : 0u) | (lx == 0 ? 2u : 0u);
    bin = ((((unsigned)(n * p.G + g) * (unsigned)p.TY + (unsigned)ty) * (unsigned)p.TX +
            (unsigned)tx) << 2) | sub;
    local = ((unsigned)ly << 4) | (unsigned)lx;
    return true;
}

// Block-level aggregation of bin counters: an LDS hash table (open addressing,
// kHash slots) from bin to a local count. block_bin_slot() inserts a sample's bin
// and returns its slot and its rank among the block's samples of that bin (the
// integer LDS atomics used here are fast); a full table returns kHash and the
// caller falls back to a global atomic for that sample.
constexpr int kHash = 256;
constexpr unsigned kEmpty = 0xffffffffu;

__device__ __forceinline__ int hash_insert(unsigned *s_key, unsigned bin) {
    unsigned h = (bin * 2654435761u) >> 24;
    for (int probe = 0; probe < kHash; ++probe) {
        const unsigned cur = atomicCAS(&s_key[h], kEmpty, bin);
        if (cur == kEmpty || cur == bin) return (int)h;
        h = (h + 1) & (kHash - 1);
    }
    return kHash;
}

// Slot of `bin` in the table and the sample's rank among the block's samples of
// that bin (kHash when the table is full). Callers spread a block's samples over
// its lanes tap-fastest, so the lanes of one instruction mostly hold different
// bins and rarely contend on one LDS word.
__device__ __forceinline__ int block_bin_slot(unsigned *s_key, unsigned *s_cnt, unsigned bin,
                                              unsigned &rank) {
    const int slot = hash_insert(s_key, bin);
    if (slot < kHash) rank = atomicAdd(&s_cnt[slot], 1u);
    return slot;
}

// Bins near a block's output tile are counted in a directly indexed LDS window
// instead of the hash table: kWin x kWin input tiles (x 4 sub-bins) around the tile
// holding the grid base of the output tile's first pixel, which covers the taps of
// a stride-1 3x3 tile with offsets up to about +-16 px. Other bins use the table.
constexpr int kWin = 5;
constexpr int kWinSlots = kWin * kWin * 4;

__device__ __forceinline__ int floor_div16(int v) { return v >= 0 ? v / kBinTile : -((-v + kBinTile - 1) / kBinTile); }

struct BinWin {
    int ty0, tx0;  // first input-tile row / column of the window
};

template <class P>
__device__ __forceinline__ BinWin bin_window(int ho0, int wo0, const P &p) {
    BinWin w;
    w.ty0 = floor_div16(ho0 * p.sh - p.ph + 1) - 2;
    w.tx0 = floor_div16(wo0 * p.sw - p.pw + 1) - 2;
    return w;
}

// Window slot of a home bin (its tile and sub-bin from home_bin's arithmetic), or -1.
__device__ __forceinline__ int win_slot(int y0, int x0, const BinWin &w) {
    const int ty = (y0 + 1) / kBinTile, tx = (x0 + 1) / kBinTile;  // y0, x0 >= -1 here
    const int wy = ty - w.ty0, wx = tx - w.tx0;
    if ((unsigned)wy >= (unsigned)kWin || (unsigned)wx >= (unsigned)kWin) return -1;
    const int ly = y0 + 1 - ty * kBinTile, lx = x0 + 1 - tx * kBinTile;
    const int sub = (ly == 0 ? 1 : 0) | (lx == 0 ? 2 : 0);
    return (wy * kWin + wx) * 4 + sub;
}

// The global bin of window slot s for (image n, group g).
template <class P>
__device__ __forceinline__ unsigned win_bin(int s, int n, int g, const BinWin &w, const P &p) {
    const int sub = s & 3, t = s >> 2;
    const int ty = w.ty0 + t / kWin, tx = w.tx0 + t % kWin;
    return ((((unsigned)(n * p.G + g) * (unsigned)p.TY + (unsigned)ty) * (unsigned)p.TX + (unsigned)tx)
            << 2) | (unsigned)sub;
}

