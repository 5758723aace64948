// Work partitioner for ragged prefill (host only, no HIP calls).
//
// The pages plan once per batch from qo_indptr / kv_indptr and run once per
// layer ("vllm.v1.attention.backends.mla.prefill.flashinfer",
// finalize_attention_metadata: plan() with kv_indptr = qo_indptr for the
// causal pass and kv_indptr = cu_seq_lens[i] for each context chunk).
// This partitioner turns those indptrs into work items, ordered for the
// MI355X:
//
//  1. A sequence is cut into query tiles of `block_m` rows. A tile needs keys
//     [0, kv_hi) of its sequence, kv_hi from the bottom-right causal rule (or
//     kv_len when non-causal); its cost per head is kv_hi plus a fixed charge
//     for loading Q and writing O.
//  2. One work item is one query tile for a block of consecutive heads
//     (one head unless the caller asks for more): the kernel runs the heads
//     one after the other with its K/V pipeline streaming straight from one
//     head into the next.
//  3. All tiles of one (sequence, head block) form a group: they read the
//     same K/V rows, so they should share one XCD's L2. Groups are dealt to
//     the XCD bins heaviest first, each to the currently lightest bin (LPT).
//  4. Each bin lists its groups heaviest first and, inside a group, its
//     tiles heaviest first, so long tiles start early and the tail is short.
//  5. The hardware hands workgroup i to XCD i mod n_xcd, so bin x's s-th
//     workgroup is placed at slot s * n_xcd + x; shorter bins are padded
//     with empty items (n_rows = 0) that the kernel skips.
//  6. Optionally (pair_max_keys > 0) a workgroup runs two items back to
//     back, the K/V pipeline streaming from the first into the second, so
//     a workgroup's fixed cost (Q load, pipeline fill and drain, the
//     hardware's dispatch of a workgroup) is paid once for both:
//     - going up from a sequence's lightest tile, two neighbouring tiles
//       are paired while the keys they see add up to at most
//       pair_max_keys (the light tiles of a causal sequence, where that
//       cost is a large share); heavy causal tiles stay alone, so the
//       units the tail is balanced with stay fine-grained;
//     - a sequence whose tiles all see the same keys (non-causal) is cut
//       into pairs of neighbouring tiles when it has at least
//       kPairEqualMinTiles tiles and at most kPairEqualMaxKeys keys: its
//       group then still runs several workgroups side by side over K/V
//       that L2 holds (with few tiles over long keys, pairs halve that
//       sharing and read the keys twice from HBM).
//     Pairing is only used for batches of like sequences (every non-empty
//     sequence within kPairMaxTilesPerSeq query tiles, the longest query and
//     key lengths at most 1.5 times the shortest): the kernel form that runs
//     two items is ~2-4% slower per tile than the one-item form (measured on
//     MI355X with identical loop code; the compiler places the running-max
//     chain differently), which pairing repays on such batches (+1 to +10%)
//     but not on batches of mixed or long sequences (-1 to -4%).
//     If any pair forms, the list holds two entries per workgroup slot
//     (the second one empty for a lone tile), else one.
#include <algorithm>
#include <climits>
#include <numeric>

#include "internal.h"

namespace mla {

namespace {
constexpr int64_t kTileFixedCost = 64;   // Q load + epilogue, in key-equivalents
// equal-tile pairing (measured on MI355X, non-causal bf16 batches, against
// light pairs only: +3 to +12% at 8-16 tiles per sequence over 1024-4096
// keys; with 4 tiles over 8192 keys pairing lost 10%, with 16 over 8192 2%)
constexpr size_t kPairEqualMinTiles = 8;
constexpr int32_t kPairEqualMaxKeys = 4096;
constexpr int64_t kPairMaxTilesPerSeq = 32;

// Whether the batch is one that pairing pays on (step 6): non-empty
// sequences of at most kPairMaxTilesPerSeq query tiles whose longest query
// and key lengths are within 1.5 times the shortest.
bool pairing_pays(const int32_t* qo, const int32_t* kv, int batch, int block_m) {
    int64_t q_min = INT64_MAX, q_max = 0, k_min = INT64_MAX, k_max = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t ql = qo[b + 1] - qo[b], kl = kv[b + 1] - kv[b];
        if (ql == 0) continue;
        q_min = std::min(q_min, ql);
        q_max = std::max(q_max, ql);
        k_min = std::min(k_min, kl);
        k_max = std::max(k_max, kl);
    }
    if (q_max == 0) return false;
    if ((q_max + block_m - 1) / block_m > kPairMaxTilesPerSeq) return false;
    return 2 * q_max <= 3 * q_min && 2 * k_max <= 3 * k_min;
}

struct Tile {
    int32_t q_row0, n_rows, kv_start, kv_len, diag0, kv_hi, seq;
    int64_t cost;
};
}  // namespace

bool build_work_list(const int32_t* qo, const int32_t* kv, int batch, int num_heads,
                     bool causal, int block_m, int n_xcd, int heads_per_item,
                     std::vector<WorkItem>& out, std::string& err, bool kv_start_is_seq,
                     int pair_max_keys, int* items_per_wg) {
    out.clear();
    if (items_per_wg != nullptr) *items_per_wg = 1;
    if (batch < 0) { err = "batch must be >= 0"; return false; }
    if (num_heads < 1 || num_heads > 65535) { err = "num_heads must be in [1, 65535]"; return false; }
    if (block_m < 1) { err = "block_m must be >= 1"; return false; }
    if (n_xcd < 1 || n_xcd > 64) { err = "n_xcd must be in [1, 64]"; return false; }
    if (pair_max_keys < 0) { err = "pair_max_keys must be >= 0"; return false; }
    if (heads_per_item < 0 || (heads_per_item > 0 && num_heads % heads_per_item != 0)) {
        err = "heads_per_item must be 0 (automatic) or divide num_heads";
        return false;
    }
    if (batch == 0) return true;
    if (qo == nullptr || kv == nullptr) { err = "indptr pointer is NULL"; return false; }
    if (qo[0] != 0 || kv[0] != 0) { err = "indptr[0] must be 0"; return false; }
    for (int b = 0; b < batch; ++b) {
        if (qo[b + 1] < qo[b]) { err = "qo_indptr must be non-decreasing"; return false; }
        if (kv[b + 1] < kv[b]) { err = "kv_indptr must be non-decreasing"; return false; }
    }

    // Tiles of every sequence (shared by all heads).
    std::vector<Tile> tiles;
    std::vector<std::pair<size_t, size_t>> seq_tiles(batch);   // [begin, end) into tiles
    for (int b = 0; b < batch; ++b) {
        const int32_t qo_len = qo[b + 1] - qo[b];
        const int32_t kv_len = kv[b + 1] - kv[b];
        const size_t begin = tiles.size();
        for (int32_t r0 = 0; r0 < qo_len; r0 += block_m) {
            Tile t;
            t.q_row0 = qo[b] + r0;
            t.n_rows = std::min(block_m, qo_len - r0);
            t.kv_start = kv_start_is_seq ? b : kv[b];
            t.kv_len = kv_len;
            // row r sees keys < kv_len - qo_len + (r0 + r) + 1 when causal
            t.diag0 = causal ? kv_len - qo_len + r0 : kv_len;
            const int64_t lim_last = static_cast<int64_t>(t.diag0) + t.n_rows;
            t.kv_hi = static_cast<int32_t>(std::min<int64_t>(kv_len, std::max<int64_t>(0, lim_last)));
            t.seq = b;
            t.cost = t.kv_hi + kTileFixedCost;
            tiles.push_back(t);
        }
        seq_tiles[b] = {begin, tiles.size()};
        // heaviest tile first inside the sequence
        std::stable_sort(tiles.begin() + begin, tiles.end(),
                         [](const Tile& a, const Tile& c) { return a.cost > c.cost; });
    }
    if (tiles.empty()) return true;

    // Head blocks are a caller's choice; measured on MI355X, one head per
    // item is never slower at the MLA shapes (the next head's Q load cannot be
    // issued early enough to hide its latency, and bigger items balance worse).
    const int nh = heads_per_item == 0 ? 1 : heads_per_item;
    const int n_blocks = num_heads / nh;

    // Groups = (sequence, head block); all blocks of a sequence cost the same.
    struct Group { int32_t seq, head0; int64_t cost; };
    std::vector<Group> groups;
    groups.reserve(static_cast<size_t>(batch) * n_blocks);
    for (int b = 0; b < batch; ++b) {
        if (seq_tiles[b].first == seq_tiles[b].second) continue;
        int64_t c = 0;
        for (size_t i = seq_tiles[b].first; i < seq_tiles[b].second; ++i) c += tiles[i].cost;
        for (int hb = 0; hb < n_blocks; ++hb) groups.push_back({b, hb * nh, c * nh});
    }
    std::stable_sort(groups.begin(), groups.end(),
                     [](const Group& a, const Group& c) { return a.cost > c.cost; });

    if (pair_max_keys > 0 && !pairing_pays(qo, kv, batch, block_m)) pair_max_keys = 0;

    // Workgroup units of every sequence: one tile, or a pair of light tiles
    // (the lighter one first); heaviest unit first. -1 marks no second tile.
    struct Unit { int64_t first, second, cost; };
    std::vector<std::vector<Unit>> seq_units(batch);
    bool any_pair = false;
    for (int b = 0; b < batch; ++b) {
        const size_t begin = seq_tiles[b].first, m = seq_tiles[b].second - begin;
        std::vector<Unit>& u = seq_units[b];
        const bool equal = pair_max_keys > 0 && m >= kPairEqualMinTiles &&
                           tiles[begin].kv_hi > 0 && tiles[begin].kv_hi == tiles[begin + m - 1].kv_hi &&
                           tiles[begin].kv_len <= kPairEqualMaxKeys;
        if (equal) {
            // equal costs keep the query order: pair tiles 2k and 2k + 1
            for (size_t k = 0; k + 1 < m; k += 2) {
                const int64_t t = static_cast<int64_t>(begin + k);
                u.push_back({t, t + 1, tiles[t].cost + tiles[t + 1].cost});
            }
            if (m % 2) u.push_back({static_cast<int64_t>(begin + m - 1), -1, tiles[begin + m - 1].cost});
            any_pair = true;
            std::stable_sort(u.begin(), u.end(),
                             [](const Unit& a, const Unit& c) { return a.cost > c.cost; });
            continue;
        }
        // tiles are sorted heaviest first: walk from the lightest (index m-1)
        size_t i = m;
        while (i > 0) {
            const int64_t t = static_cast<int64_t>(begin + i - 1);
            if (pair_max_keys > 0 && i >= 2) {
                const int64_t t2 = t - 1;
                if (static_cast<int64_t>(tiles[t].kv_hi) + tiles[t2].kv_hi <= pair_max_keys) {
                    u.push_back({t, t2, tiles[t].cost + tiles[t2].cost});
                    any_pair = true;
                    i -= 2;
                    continue;
                }
            }
            u.push_back({t, -1, tiles[t].cost});
            i -= 1;
        }
        std::stable_sort(u.begin(), u.end(),
                         [](const Unit& a, const Unit& c) { return a.cost > c.cost; });
    }
    const size_t per_wg = any_pair ? 2 : 1;
    if (items_per_wg != nullptr) *items_per_wg = static_cast<int>(per_wg);

    // LPT deal into XCD bins.
    std::vector<std::vector<const Group*>> bins(n_xcd);
    std::vector<int64_t> load(n_xcd, 0);
    std::vector<size_t> count(n_xcd, 0);
    for (const Group& g : groups) {
        int best = 0;
        for (int x = 1; x < n_xcd; ++x)
            if (load[x] < load[best]) best = x;
        bins[best].push_back(&g);
        load[best] += g.cost;
        count[best] += seq_units[g.seq].size();
    }
    const size_t slots = *std::max_element(count.begin(), count.end());

    WorkItem pad{};
    out.assign(slots * static_cast<size_t>(n_xcd) * per_wg, pad);
    auto put = [&](size_t at, const Tile& t, int32_t head0) {
        WorkItem& w = out[at];
        w.q_row0 = t.q_row0;
        w.n_rows = t.n_rows;
        w.head0 = head0;
        w.n_heads = nh;
        w.kv_start = t.kv_start;
        w.kv_len = t.kv_len;
        w.diag0 = t.diag0;
        w.kv_hi = t.kv_hi;
    };
    for (int x = 0; x < n_xcd; ++x) {
        size_t s = 0;
        for (const Group* g : bins[x]) {
            for (const Unit& u : seq_units[g->seq]) {
                const size_t at = (s * n_xcd + x) * per_wg;
                put(at, tiles[u.first], g->head0);
                if (u.second >= 0) put(at + 1, tiles[u.second], g->head0);
                ++s;
            }
        }
    }
    return true;
}

// Weight-absorbed prefill: every head of a token reads the same latent
// cache rows, so a sequence's work is its flat (token, head) rows cut into
// tiles of block_m rows. Groups are runs of at most kLatentGroupTiles
// consecutive tiles of one sequence (heaviest tiles first), so a long
// sequence spreads over several XCDs while each group still shares one L2;
// groups are dealt and laid out exactly as above. With KV splits every tile
// becomes `splits` items over consecutive ranges of its 32-key tiles.
namespace {
constexpr int kLatentKeyTile = 32;
}  // namespace

int latent_kv_splits(const int32_t* qo, const int32_t* kv, int batch, int num_heads, bool causal,
                     int block_m) {
    // One workgroup fits a CU, so the target is one item per CU in a single
    // round: split only when the row tiles are fewer than the CUs, up to 32
    // ways while each split keeps at least 4 key tiles. (Measured on MI355X
    // for a decode step of 64 requests over 4096-token caches: 4 splits in
    // one round 0.126-0.133 ms, 8 in two rounds 0.156-0.159 ms, 16 in four
    // 0.23 ms; each item's fixed cost outweighs the finer balance.)
    constexpr int64_t kTargetItems = 256;
    constexpr int kMaxSplits = 32, kMinTilesPerSplit = 4;
    if (batch <= 0 || qo == nullptr || kv == nullptr || num_heads < 1 || block_m < 1) return 1;
    int64_t row_tiles = 0, max_key_tiles = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t qo_len = qo[b + 1] - qo[b], kv_len = kv[b + 1] - kv[b];
        if (qo_len <= 0 || kv_len <= 0) continue;
        row_tiles += (qo_len * num_heads + block_m - 1) / block_m;
        // the last row of the sequence sees the most keys
        const int64_t diag = causal ? kv_len - qo_len : kv_len;
        int64_t lim = diag + qo_len;
        lim = lim < 0 ? 0 : (lim > kv_len ? kv_len : lim);
        const int64_t t = (lim + kLatentKeyTile - 1) / kLatentKeyTile;
        max_key_tiles = t > max_key_tiles ? t : max_key_tiles;
    }
    if (row_tiles == 0 || row_tiles >= kTargetItems) return 1;
    int64_t s = (kTargetItems + row_tiles - 1) / row_tiles;
    s = s > kMaxSplits ? kMaxSplits : s;
    const int64_t by_len = max_key_tiles / kMinTilesPerSplit;
    s = s > by_len ? by_len : s;
    return s < 1 ? 1 : static_cast<int>(s);
}

bool build_latent_work_list(const int32_t* qo, const int32_t* kv, int batch, int num_heads,
                            bool causal, int block_m, int n_xcd, std::vector<LatentItem>& out,
                            std::string& err, bool kv_start_is_seq, int splits) {
    constexpr size_t kLatentGroupTiles = 256;
    out.clear();
    if (batch < 0) { err = "batch must be >= 0"; return false; }
    if (num_heads < 1 || num_heads > 65535) { err = "num_heads must be in [1, 65535]"; return false; }
    if (block_m < 1) { err = "block_m must be >= 1"; return false; }
    if (n_xcd < 1 || n_xcd > 64) { err = "n_xcd must be in [1, 64]"; return false; }
    if (splits < 1 || splits > 64) { err = "splits must be in [1, 64]"; return false; }
    if (batch == 0) return true;
    if (qo == nullptr || kv == nullptr) { err = "indptr pointer is NULL"; return false; }
    if (qo[0] != 0 || kv[0] != 0) { err = "indptr[0] must be 0"; return false; }
    for (int b = 0; b < batch; ++b) {
        if (qo[b + 1] < qo[b]) { err = "qo_indptr must be non-decreasing"; return false; }
        if (kv[b + 1] < kv[b]) { err = "kv_indptr must be non-decreasing"; return false; }
    }
    if (static_cast<int64_t>(qo[batch]) * num_heads > 0x7fffffffLL) {
        err = "total query rows (tokens x heads) must be < 2^31";
        return false;
    }

    struct LTile { LatentItem item; int64_t cost; };
    std::vector<LTile> tiles;
    struct Group { size_t begin, end; int64_t cost; };
    std::vector<Group> groups;
    for (int b = 0; b < batch; ++b) {
        const int32_t qo_len = qo[b + 1] - qo[b];
        const int32_t kv_len = kv[b + 1] - kv[b];
        const int32_t seq_row0 = qo[b] * num_heads;
        const int32_t n_rows_seq = qo_len * num_heads;
        const int32_t diag_base = causal ? kv_len - qo_len : kv_len;
        const size_t begin = tiles.size();
        for (int32_t r0 = 0; r0 < n_rows_seq; r0 += block_m) {
            LTile t{};
            t.item.row0 = seq_row0 + r0;
            t.item.n_rows = std::min(block_m, n_rows_seq - r0);
            t.item.seq_row0 = seq_row0;
            const int64_t last_tok = (r0 + t.item.n_rows - 1) / num_heads;
            const int64_t lim_last = static_cast<int64_t>(diag_base) + last_tok + 1;
            const int32_t kv_hi =
                static_cast<int32_t>(std::min<int64_t>(kv_len, std::max<int64_t>(0, lim_last)));
            t.item.kv_start = kv_start_is_seq ? b : kv[b];
            t.item.kv_len = kv_len;
            t.item.diag_base = diag_base;
            const int32_t key_tiles = (kv_hi + kLatentKeyTile - 1) / kLatentKeyTile;
            for (int s = 0; s < splits; ++s) {
                const int32_t t0 = static_cast<int32_t>(static_cast<int64_t>(key_tiles) * s / splits);
                const int32_t t1 = static_cast<int32_t>(static_cast<int64_t>(key_tiles) * (s + 1) / splits);
                t.item.kv_lo = t0 * kLatentKeyTile;
                t.item.kv_hi = s + 1 == splits ? kv_hi : std::min(kv_hi, t1 * kLatentKeyTile);
                if (t.item.kv_hi < t.item.kv_lo) t.item.kv_hi = t.item.kv_lo;
                t.item.part = splits > 1 ? s : -1;
                t.cost = (t.item.kv_hi - t.item.kv_lo) + kTileFixedCost;
                tiles.push_back(t);
            }
        }
        std::stable_sort(tiles.begin() + begin, tiles.end(),
                         [](const LTile& a, const LTile& c) { return a.cost > c.cost; });
        for (size_t g0 = begin; g0 < tiles.size(); g0 += kLatentGroupTiles) {
            const size_t g1 = std::min(tiles.size(), g0 + kLatentGroupTiles);
            int64_t c = 0;
            for (size_t i = g0; i < g1; ++i) c += tiles[i].cost;
            groups.push_back({g0, g1, c});
        }
    }
    if (tiles.empty()) return true;
    std::stable_sort(groups.begin(), groups.end(),
                     [](const Group& a, const Group& c) { return a.cost > c.cost; });

    std::vector<std::vector<const Group*>> bins(n_xcd);
    std::vector<int64_t> load(n_xcd, 0);
    std::vector<size_t> count(n_xcd, 0);
    for (const Group& g : groups) {
        int best = 0;
        for (int x = 1; x < n_xcd; ++x)
            if (load[x] < load[best]) best = x;
        bins[best].push_back(&g);
        load[best] += g.cost;
        count[best] += g.end - g.begin;
    }
    const size_t slots = *std::max_element(count.begin(), count.end());
    out.assign(slots * static_cast<size_t>(n_xcd), LatentItem{});
    for (int x = 0; x < n_xcd; ++x) {
        size_t s = 0;
        for (const Group* g : bins[x])
            for (size_t i = g->begin; i < g->end; ++i, ++s) out[s * n_xcd + x] = tiles[i].item;
    }
    return true;
}

}  // namespace mla
