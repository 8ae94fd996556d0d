// Test driver for the library's host-side rules (block_quant_weight_amd/
// csrc/qmv_host.cpp, no HIP), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitize_cpu.py.  Reads one case
// per line from stdin and prints one result line per case:
//   span WT SF ROWS COLS                -> status q_bytes d_offset d_bytes min_span
//   gspan WT ROWS COLS                  -> status bytes
//   class FW MASK BIT SHARED            -> status wtype
//   check WT SF ROWS COLS NBYTES PLANT  -> status of check_bytes on NBYTES zero
//                                          bytes (exactly that many allocated)
//                                          with 0x80 at PLANT (if in range)
//   gcheck WT ROWS COLS NBYTES PLANT    -> status of check_gguf, the same way
//   exps WT SF ROWS COLS GGUF SEED      -> the matrix exponent and every row
//                                          exponent of scale_exponents over
//                                          seeded scale bits
//   status K                            -> the status text
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "qmv.h"
#include "qmv_layout.h"

namespace {

// splitmix64: the seeded bits of the scale arrays
uint64_t next(uint64_t& s) {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// An exact-size heap copy, so that any read past nbytes is caught.
uint8_t* zeros(uint64_t nbytes, int64_t plant) {
    uint8_t* p = static_cast<uint8_t*>(std::malloc(nbytes ? nbytes : 1));
    std::memset(p, 0, nbytes);
    if (plant >= 0 && static_cast<uint64_t>(plant) < nbytes) p[plant] = 0x80;
    return p;
}

}  // namespace

int main() {
    char cmd[16];
    while (std::scanf("%15s", cmd) == 1) {
        const std::string c(cmd);
        if (c == "span") {
            unsigned wt, sf, r, k;
            if (std::scanf("%u %u %u %u", &wt, &sf, &r, &k) != 4) return 2;
            uint64_t a = 0, b = 0, d = 0, m = 0;
            const int st = qmv_span(wt, sf, r, k, &a, &b, &d, &m);
            std::printf("%d %llu %llu %llu %llu\n", st, (unsigned long long)a, (unsigned long long)b,
                        (unsigned long long)d, (unsigned long long)m);
        } else if (c == "gspan") {
            unsigned wt, r, k;
            if (std::scanf("%u %u %u", &wt, &r, &k) != 3) return 2;
            uint64_t n = 0;
            const int st = qmv_gguf_span(wt, r, k, &n);
            std::printf("%d %llu\n", st, (unsigned long long)n);
        } else if (c == "class") {
            unsigned fw, mask, bit, shared;
            if (std::scanf("%u %u %u %u", &fw, &mask, &bit, &shared) != 4) return 2;
            uint32_t w = 0;
            const int st = qmv_class_wtype(fw, mask, bit, shared, &w);
            std::printf("%d %u\n", st, w);
        } else if (c == "check" || c == "gcheck") {
            const bool g = c == "gcheck";
            unsigned wt, sf = 1, r, k;
            unsigned long long nbytes;
            long long plant;
            if (g) {
                if (std::scanf("%u %u %u %llu %lld", &wt, &r, &k, &nbytes, &plant) != 5) return 2;
            } else {
                if (std::scanf("%u %u %u %u %llu %lld", &wt, &sf, &r, &k, &nbytes, &plant) != 6) return 2;
            }
            qmv::Layout L;
            int st = qmv::compute_layout(wt, sf, r, k, &L);
            if (st == QMV_OK) {
                uint8_t* p = zeros(nbytes, plant);
                st = g ? qmv::check_gguf(L, p, nbytes) : qmv::check_bytes(L, p, nbytes);
                std::free(p);
            }
            std::printf("%d\n", st);
        } else if (c == "exps") {
            unsigned wt, sf, r, k, g;
            unsigned long long seed;
            if (std::scanf("%u %u %u %u %u %llu", &wt, &sf, &r, &k, &g, &seed) != 6) return 2;
            qmv::Layout L;
            if (qmv::compute_layout(wt, g ? 1 : sf, r, k, &L) != QMV_OK) {
                std::printf("layout\n");
                continue;
            }
            uint64_t s = seed;
            uint64_t n = L.min_span;
            if (g) {
                uint64_t gb = 0;
                if (qmv::gguf_bytes(wt, r, k, &gb) != QMV_OK) return 3;
                n = gb;
            }
            std::vector<uint8_t> buf(n);
            for (auto& v : buf) v = static_cast<uint8_t>(next(s));
            std::vector<int32_t> rows(r);
            int32_t all = -999;
            qmv::scale_exponents(L, buf.data(), g != 0, rows.data(), &all);
            std::printf("%d", all);
            for (int32_t e : rows) std::printf(" %d", e);
            std::printf("\n");
        } else if (c == "status") {
            int k;
            if (std::scanf("%d", &k) != 1) return 2;
            std::printf("%s\n", qmv_status_str(k));
        } else {
            return 2;
        }
    }
    return 0;
}
