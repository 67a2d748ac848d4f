// Host driver for the checkpoint file module (zsp_ckpt.cpp), built with g++
// and AddressSanitizer / UBSan by tests/test_ckpt_sanitized.py. It writes rank
// files, maps and checks them, then feeds the reader truncated, bit-flipped
// and hostile files: every one must be refused with an error status, and
// nothing may read or allocate out of bounds. A file replaced by rename after
// its check must not change what the mapping reads. Prints "ok" at the end.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <string>
#include <vector>

#include "zsp_ckpt.hpp"

using namespace zsp;

static int failures = 0;
#define EXPECT(c)                                                       \
    do {                                                                \
        if (!(c)) {                                                     \
            std::printf("FAIL line %d: %s\n", __LINE__, #c);            \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static std::string path_of(const std::string& dir, int r, int nd) {
    return dir + "/rank-" + std::to_string(r) + "-of-" + std::to_string(nd) + ".zsp";
}

static std::vector<char> slurp(const std::string& p) {
    std::ifstream f(p, std::ios::binary);
    return std::vector<char>((std::istreambuf_iterator<char>(f)), std::istreambuf_iterator<char>());
}

static void spill(const std::string& p, const char* data, size_t n) {
    std::ofstream f(p, std::ios::binary | std::ios::trunc);
    f.write(data, std::streamsize(n));
}

static CkptStatus verify(const std::string& dir, int nd, int r, std::vector<int64_t>* numel,
                         int64_t* S, int64_t* step) {
    MappedRank m;
    std::string err;
    return m.open(dir.c_str(), nd, r, numel, S, step, &err);
}

int main(int argc, char** argv) {
    if (argc != 2) return 2;
    const std::string dir = argv[1];
    const int nd = 4;
    const std::vector<int64_t> numel = {1003, 64, 5, 0, 12289, 7};
    int64_t S = 0;
    for (int64_t n : numel) S += (n + (nd - n % nd) % nd) / nd;

    // round trip of every rank
    std::vector<std::vector<float>> ma(nd), mm(nd), mv(nd);
    std::vector<std::vector<uint16_t>> mw(nd);
    uint32_t seed = 12345;
    auto next = [&] { seed = seed * 1664525u + 1013904223u; return seed; };
    for (int r = 0; r < nd; ++r) {
        ma[r].resize(S); mm[r].resize(S); mv[r].resize(S); mw[r].resize(S);
        for (int64_t i = 0; i < S; ++i) {
            ma[r][i] = float(next() % 1000) * 0.5f;
            mm[r][i] = float(next() % 1000) * 0.25f;
            mv[r][i] = float(next() % 1000) * 0.125f;
            mw[r][i] = uint16_t(next());
        }
        HostPayload src(ma[r].data(), mm[r].data(), mv[r].data(), mw[r].data(), S);
        std::string err;
        EXPECT(ckpt_write_rank(dir.c_str(), nd, r, numel, S, 42, src, &err) == CkptStatus::Ok);
    }
    EXPECT(ckpt_find_nd(dir.c_str()) == nd);
    for (int r = 0; r < nd; ++r) {
        std::vector<int64_t> got;
        int64_t s = -1, step = -1;
        MappedRank m;
        std::string err;
        EXPECT(m.open(dir.c_str(), nd, r, &got, &s, &step, &err) == CkptStatus::Ok);
        EXPECT(got == numel && s == S && step == 42);
        EXPECT(std::memcmp(m.master(), ma[r].data(), size_t(S) * 4) == 0);
        EXPECT(std::memcmp(m.m(), mm[r].data(), size_t(S) * 4) == 0);
        EXPECT(std::memcmp(m.v(), mv[r].data(), size_t(S) * 4) == 0);
        EXPECT(std::memcmp(m.work(), mw[r].data(), size_t(S) * 2) == 0);
    }

    // damaged copies of rank 1
    const std::string p1 = path_of(dir, 1, nd);
    const std::vector<char> good = slurp(p1);
    const size_t len = good.size();
    std::vector<int64_t> got;
    int64_t s = 0, step = 0;
    const size_t cuts[] = {0, 1, 7, 8, 47, 48, 55, 56, len / 2, len - 9, len - 8, len - 1};
    for (size_t c : cuts) {
        spill(p1, good.data(), c);
        EXPECT(verify(dir, nd, 1, &got, &s, &step) == CkptStatus::Corrupt);
    }
    std::vector<char> longer(good);
    longer.push_back(0);
    spill(p1, longer.data(), longer.size());
    EXPECT(verify(dir, nd, 1, &got, &s, &step) == CkptStatus::Corrupt);
    for (size_t i = 0; i < len; i += (i < 128 ? 1 : 97)) {  // every header byte, then a sample
        for (int bit : {0, 6}) {
            std::vector<char> bad(good);
            bad[i] = char(bad[i] ^ (1 << bit));
            spill(p1, bad.data(), bad.size());
            EXPECT(verify(dir, nd, 1, &got, &s, &step) == CkptStatus::Corrupt);
        }
    }
    // hostile header fields in a short file: huge T, huge S, negative S
    for (int field = 2; field <= 3; ++field) {
        for (int64_t value : {int64_t(1) << 31, int64_t(1) << 40, int64_t(-1), int64_t(0)}) {
            std::vector<char> bad(good.begin(), good.begin() + 48);
            std::memcpy(bad.data() + 8 + 8 * field, &value, 8);
            spill(p1, bad.data(), bad.size());
            EXPECT(verify(dir, nd, 1, &got, &s, &step) == CkptStatus::Corrupt);
        }
    }
    spill(p1, good.data(), len);
    EXPECT(verify(dir, nd, 1, &got, &s, &step) == CkptStatus::Ok);
    std::remove(p1.c_str());
    EXPECT(verify(dir, nd, 1, &got, &s, &step) == CkptStatus::Missing);
    spill(p1, good.data(), len);

    // a file renamed over the mapped one after its check leaves the mapping,
    // and the payload read from it, as checked
    {
        std::vector<int64_t> g2;
        int64_t s2 = 0, st2 = 0;
        MappedRank m;
        std::string err;
        EXPECT(m.open(dir.c_str(), nd, 2, &g2, &s2, &st2, &err) == CkptStatus::Ok);
        HostPayload src(ma[3].data(), mm[3].data(), mv[3].data(), mw[3].data(), S);
        EXPECT(ckpt_write_rank(dir.c_str(), nd, 2, numel, S, 43, src, &err) == CkptStatus::Ok);
        EXPECT(std::memcmp(m.master(), ma[2].data(), size_t(S) * 4) == 0);
        EXPECT(std::memcmp(m.work(), mw[2].data(), size_t(S) * 2) == 0);
    }

    // directory scans: junk names are ignored, two rank counts are refused
    spill(dir + "/rank-x-of-4.zsp", "", 0);
    spill(dir + "/rank-9-of-4.zsp", "", 0);
    spill(dir + "/rank-0-of-4.zsp.tmp", "", 0);
    EXPECT(ckpt_find_nd(dir.c_str()) == nd);
    spill(dir + "/rank-0-of-2.zsp", "", 0);
    EXPECT(ckpt_find_nd(dir.c_str()) == -1);
    EXPECT(ckpt_find_nd((dir + "/missing").c_str()) == 0);

    if (failures == 0) std::printf("ok\n");
    return failures == 0 ? 0 : 1;
}
