// What the recording launchers (launch_record.cpp) saw.
#pragma once
#include "launch.h"

namespace mxk {

enum { kLaunchNone, kLaunchMx, kLaunchMxGrouped, kLaunchValues, kLaunchAbsmax, kLaunchNv,
       kLaunchNvGrouped, kLaunchAbsmaxGrouped, kLaunchMxAny, kLaunchValuesAny, kLaunchNvAny,
       kLaunchMxRagged, kLaunchNvRagged };

struct Record {
    int calls = 0, reduces = 0, kind = kLaunchNone;
    int op = 0, segments = 0;
    unsigned axis = 0, fmt = 0;
    bool dbias = false, two_d = false;
    int64_t M = 0, K = 0;
    MxArgs mx{};
    Nv4Args nv{};
    GroupTable gt{};
};

extern Record g_rec;

}  // namespace mxk
