// kvp_plan_format.h -- layout of a decode work plan (internal to the library; the host
// planner writes it, the fp16 decode kernel reads it).
//
// A plan is one int32 image:
//   items       [n_items][REC]   one record per work item (= one wave of the kernel)
//   pair_base   [B * Hkv]        first partial slot of pair (b, g), -1 if the pair has one part
//   pair_nparts [B * Hkv]        parts the pair's attention row is split into (>= 1)
//   req_shared  [B]              tokens [0, req_shared[b]) of request b are read by a shared item
//   ids         [n_ids]          block ids of long items (built with KVP_PLAN_LONG_ITEMS only)
//
// A work item covers up to BPI consecutive 16-token blocks of one KV head: either of one
// request (private item) or of the leading request of a run of requests whose tables point
// at the same physical blocks there (shared item: the blocks are read once and attended by
// every member's queries, each member up to its own req_shared limit).
#pragma once

namespace kvp {
namespace plan {

constexpr int BPI = 32;  // blocks per work item (512 tokens)
// A pair (or shared unit) of at most BPI blocks is one item when nothing else splits it;
// otherwise it is cut into ceil(blocks / SPLIT_BLOCKS) parts of equal tile counts (at most
// BPI blocks each).  Shorter parts mean more waves, and the decode time grows with the wave
// count faster than the shorter tail saves, so the parts are as long as an item may be.
constexpr int SPLIT_BLOCKS = 32;
constexpr int UNSPLIT_BLOCKS = 32; // longest pair kept in one item (at most BPI)
// The int8 kernel keeps twice the waves resident (18 KB of LDS each, eight per CU): at head
// dim 64, parts of 16 blocks fill them (batch 200, 14q / 2kv: 18.6 us per launch by the trace
// against 20.6 with 32-block parts).  At head dim 128 the many more pairs already fill them
// and the extra merges cost more (32q / 8kv: 72.4 against 69.4 us), so 32 blocks stay.
constexpr int SPLIT_BLOCKS_I8_D64 = 16;
constexpr int UNSPLIT_BLOCKS_I8_D64 = 16;
constexpr int split_blocks(bool i8, int hd) { return i8 && hd == 64 ? SPLIT_BLOCKS_I8_D64 : SPLIT_BLOCKS; }
constexpr int unsplit_blocks(bool i8, int hd) { return i8 && hd == 64 ? UNSPLIT_BLOCKS_I8_D64 : UNSPLIT_BLOCKS; }
// Tiles (4 blocks) of the parts of a range of T tiles split n ways: part k covers tiles
// [part_tile_begin(T, n, k, slack), part_tile_begin(T, n, k + 1, slack)).  The last part
// -- the one that holds the range's final blocks, which merges a split pair -- gets up to
// `slack` tiles more than the others (at most 8), the others share the rest evenly.
constexpr int part_tile_begin(int T, int n, int k, int slack)
{
    if (k <= 0)
        return 0;
    if (k >= n)
        return T;
    const int even = (T + n - 1) / n;
    int m = even + slack < 8 ? even + slack : 8;
    if (m > T - (n - 1))
        m = T - (n - 1); // every other part keeps a tile
    if (m < even)
        m = even;
    const int rest = T - m;
    return k == n - 1 ? rest : (int)((long long)k * rest / (n - 1));
}
// tiles of extra length for the last part of a pair's private range (measured: giving the
// polled merge two tiles of lead over the other parts gained nothing, so none)
constexpr int SPLIT_SLACK = 0;
constexpr int REC = 48;  // int32 per record
// Long items (plans built with KVP_PLAN_LONG_ITEMS): a private range of a batch with many
// more blocks than resident waves is cut into parts of up to LONG_BPI blocks, whose ids sit
// in the image's id area (the record's first id entry holds the offset there).  Fewer,
// longer items pay the fixed start and finish of a wave fewer times.
constexpr int LONG_BPI = 192; // blocks of a long item (three ids per lane)
// waves resident at once, which a long-item plan fills about once: four 32 KB fp16
// workgroups per CU, eight of the int8 kernel's 18 KB, on 256 CUs
constexpr int LONG_TARGET_WAVES_F16 = 1024;
constexpr int LONG_TARGET_WAVES_I8 = 2048;
// shortest private part of a KVP_PLAN_FILL plan (two tiles)
constexpr int FILL_MIN_BLOCKS = 8;
constexpr int MAXM = 16; // members of one shared item
// Query columns of an item: blocks of 16 MFMA columns, at most 4 per item at head dim 64 and
// 2 at 128.  Group size G = Hq / Hkv: up to 16 (a block holds 16 / G members of G heads; a
// shared item serves up to 16 / G members per block), or a multiple of 16 (a private item
// of one request takes G / 16 blocks; no shared items).
constexpr int max_col_blocks(int hd) { return hd == 64 ? 4 : 2; }
constexpr bool group_supported(int G, int hd)
{
    return (G >= 1 && G <= 16) || (G % 16 == 0 && G / 16 <= max_col_blocks(hd));
}
// column blocks of a shared item: the plan's width (1, 2 or 4), at least 2 when a block
// holds a single member, at most max_col_blocks(hd)
constexpr int shared_col_blocks(int G, int hd, int width)
{
    const int w = G > 8 && width < 2 ? 2 : width;
    return w < max_col_blocks(hd) ? w : max_col_blocks(hd);
}
// members of one shared item at group size G (1: no shared items)
constexpr int shared_members(int G, int hd, int width)
{
    return G > 16 ? 1 : (16 / G * shared_col_blocks(G, hd, width) < MAXM ? 16 / G * shared_col_blocks(G, hd, width)
                                                                        : MAXM);
}
constexpr int XCDS = 8;  // MI355X: workgroup i runs on XCD i % 8 (round-robin dispatch)
// CUs per XCD: within an XCD, the dispatcher deals the queue positions of one launch
// round-robin over its CUs, so positions p and p + CU_SLOTS of an XCD queue share a CU
constexpr int CU_SLOTS = 32;

enum : int {
    R_FLAGS = 0,  // F_SHARED: shared item; F_EMPTY: padding, no work
    R_B = 1,      // request (private) or first member (shared)
    R_G = 2,      // KV head
    R_NMEM = 3,   // members (1 for a private item)
    R_BLK0 = 4,   // first logical block
    R_NBLK = 5,   // blocks in the item (0 only for an empty context)
    R_END = 6,    // private: context length of the request (tokens >= END are masked)
    R_SLOT = 7,   // private: partial slot written by this item (when NPARTS > 1);
                  // shared: part index inside each member's slot range
    R_NPARTS = 8, // private: parts of the pair
    R_PBASE = 9,  // private: first slot of the pair
    R_ENT = 16,   // BPI physical block ids (-1: unusable, rows masked)
};
static_assert(R_ENT + BPI <= REC, "record too small");

constexpr int F_SHARED = 1;
constexpr int F_EMPTY = 2;
constexpr int F_LONG = 4; // private item of up to LONG_BPI blocks, ids in the id area
constexpr int R_IDS = R_ENT; // long item: offset of its ids in the id area

} // namespace plan
} // namespace kvp
