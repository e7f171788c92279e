"""Double-precision CPU oracle for HLG + Gumbel-max sampling. Test infrastructure only."""
