// Workspace ownership bookkeeping (csrc/ledger.h), on the host: which plan's tables each
// workspace region holds after uploads into the same, overlapping and separate regions, and
// after plans are freed. Exits non-zero on the first wrong answer.
#include <stdio.h>
#include <stdlib.h>

#include "ledger.h"

#define CHECK(c)                                                                \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);     \
            exit(2);                                                            \
        }                                                                       \
    } while (0)

struct FakePlan {
    int id;
};

int main() {
    using piclink::WorkspaceLedger;
    static char mem[1 << 16];
    FakePlan a{1}, b{2}, c{3};
    char *w0 = mem, *w1 = mem + 4096, *w2 = mem + 8192;
    {
        WorkspaceLedger<FakePlan> L;
        CHECK(!L.holds(&a, w0));                  // never uploaded
        L.claim(&a, w0, 1024);
        CHECK(L.holds(&a, w0));
        CHECK(!L.holds(&a, w1));                  // another region
        L.claim(&b, w0, 1024);                    // B over A: A no longer held
        CHECK(L.holds(&b, w0) && !L.holds(&a, w0));
        L.claim(&a, w0, 1024);                    // A again: B dropped
        CHECK(L.holds(&a, w0) && !L.holds(&b, w0));
        CHECK(L.size() == 1);
    }
    {
        WorkspaceLedger<FakePlan> L;
        L.claim(&a, w0, 4096);                    // [w0, w0 + 4096)
        L.claim(&b, w1, 4096);                    // adjacent, no overlap
        CHECK(L.holds(&a, w0) && L.holds(&b, w1));
        L.claim(&c, w0 + 4000, 200);              // overlaps both A's end and B's start
        CHECK(!L.holds(&a, w0) && !L.holds(&b, w1) && L.holds(&c, w0 + 4000));
        L.claim(&a, w2, 100);
        L.claim(&b, w2 + 100, 100);               // touching, not overlapping
        CHECK(L.holds(&a, w2) && L.holds(&b, w2 + 100));
        L.claim(&a, w0, 100);                     // a plan holds one region: its old one ends
        CHECK(L.holds(&a, w0) && !L.holds(&a, w2) && L.holds(&b, w2 + 100));
        L.drop(&b);                               // plan freed
        CHECK(!L.holds(&b, w2 + 100) && L.holds(&a, w0));
        L.drop(&b);                               // dropping twice is harmless
        L.drop(&a);
        L.drop(&c);
        CHECK(L.size() == 0);
    }
    printf("ok\n");
    return 0;
}
